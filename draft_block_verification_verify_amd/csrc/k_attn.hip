// Rotary positions and tree-masked GQA attention for the verify step (gfx950).
//
// Rows attend to their tree's KV prefix plus their ancestors and themselves,
// with RoPE at the rows' semantic positions (onedev.kr SpecOPD summary,
// "what differs": parent map, semantic positions, ancestor-and-self mask).
//
// bf16 path: split-KV flash-decode.  A query group is (pack, KV head, up to
// 128 of the pack's (row, head-in-group) pairs), so one K/V tile streamed
// from HBM serves every row and every query head of the GQA group; a pack is
// one tree, or (head dims up to 128) consecutive trees over one KV segment,
// such as the branches of a proposal tree over a shared stem (each query
// then masks the stem past its own tree's length).  The
// tiles of all query groups, one group after another, are cut into runs of
// equal length, one per workgroup; a work item is the part of one group that
// one run covers.  K/V tiles reach LDS by DMA in their natural layout,
// V^T fragments come from transposing LDS reads, S^T = K.Q^T and
// O^T += V^T.P^T run on 16x16x32 bf16 MFMA, the online softmax is per
// wavefront in fp32 (log2 domain).  The rotated queries and the
// probabilities are each carried as a bf16 pair hi + lo (two MFMAs per
// product), so the scores of the cached keys (exact bf16 inputs) are exact
// to about 16 bits; the keys rotated in this step (the row tiles) enter the
// tiles rounded to bf16, and the merge replaces their weights with exact
// ones.  Each item leaves (max, sum, unnormalised o) per
// query; a merge kernel combines the items of a query and writes o in the
// format the W_o projection reads.
//
// fp32 path: one workgroup per (row, query head), plain fp32 arithmetic.
#include "k_common.hpp"
#include "k_dma.hpp"
#include "k_rope.hpp"
#include "launch.hpp"

namespace sv {

// RoPE launch: grid (rows, ceil(heads * d/2 / 256)); device code in k_rope.hpp.
template <typename T>
__global__ __launch_bounds__(256) void rope_rows_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                        T *__restrict__ q_out, T *__restrict__ k_out,
                                                        const int32_t *__restrict__ row_pos, int Hq,
                                                        int Hkv, int D, double base) {
  rope_rows_block<T>(q, k, q_out, k_out, row_pos, Hq, Hkv, D, base, 0, 0, blockIdx.x, blockIdx.y, gridDim.y);
}

// ----------------------------------------------------------------------------
// bf16 split-KV attention on MFMA
//
// A workgroup walks its run's tiles of KT = 8192 / D keys (16 KB of K plus
// 16 KB of V), item after item, through an STG-stage LDS ring filled by
// direct global -> LDS DMA, STG - 1 tiles ahead of the one being used; the
// DMA side crosses into the next item on its own, and the compute side
// writes an item's partial records and loads the next item's queries as it
// finishes the item's last tile.  A tile holds its keys in natural [key][d]
// layout; 16-B chunk c of tile row r sits at chunk c ^ swz(r), which keeps
// both the K fragment reads (16 rows, one chunk) and the transposing V reads
// (4 rows x 32 B per 16 lanes) free of bank conflicts.  Wavefront w owns
// query block w (16 query vectors); every wavefront issues its share of the
// DMA.  Prefix tiles come from the KV cache, row tiles from the rotated row
// keys and the row values; each DMA is range-checked against the tree's own
// keys, so padding rows read as zeros and are masked.
// ----------------------------------------------------------------------------

template <int D>
struct AttnTile {
  static constexpr int KT = attn_key_tile(D);   // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per key row
  static constexpr int TILEB = KT * ROWB;       // 16 KB
  static constexpr int CH = D / 8;              // 16-B chunks per row
  static constexpr int RPI = 1024 / ROWB;       // rows per wave DMA instruction
  static constexpr int NI = TILEB / 1024;       // DMA instructions per K (or V) tile
};
template <int D, int STG>
constexpr size_t attn_lds_bytes() { return size_t(STG) * 2 * AttnTile<D>::TILEB; }

// LDS chunk slot of logical 16-B chunk c in tile row r.  D >= 128: any 16
// aligned consecutive rows get 16 distinct slots (and any 8 rows distinct
// slots mod 8), any 8 aligned rows get 8 distinct chunk pairs; D = 64 (8
// chunks per row): 8 rows distinct, 4 aligned rows distinct pairs.
template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (D >= 128)
    return c ^ (((r & 7) << 1) | (((r >> 2) ^ (r >> 3)) & 1));
  else
    return c ^ (((r & 3) << 1) | ((r >> 2) & 1));
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j receives 16-bit element (j & 3) of the 8-byte rows addressed by
// lanes 4k + (j >> 2), k = 0..3, in that order.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t *p) {
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4 *)((__attribute__((address_space(3))) uint8_t *)(p)));
  return __builtin_bit_cast(uint2, v);
}

// Work-list records through the constant address space: the compiler then
// reads them with scalar loads (counted apart from the vector-memory loads
// whose count the DMA ring waits on) and keeps the fields in SGPRs.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *as_const(const T *p) {
  return reinterpret_cast<const __attribute__((address_space(4))) T *>(reinterpret_cast<uintptr_t>(p));
}

// STG: ring stages (tiles in flight = STG - 1); OCC: wavefronts per SIMD the
// launch is built for (registers per wavefront <= 512 / OCC); NTP: partial o
// records stored with the non-temporal hint (a template choice: as a runtime
// branch the compiler merged the two stores and dropped the hint).
template <int D, int NW, int STG, int OCC, bool NTP>
__global__ __launch_bounds__(64 * NW, OCC) void attn_mfma_kernel(AttnArgs a) {
  using TL = AttnTile<D>;
  constexpr int KT = TL::KT, ROWB = TL::ROWB, TILEB = TL::TILEB, CH = TL::CH, RPI = TL::RPI;
  constexpr int DS = D / 32;      // 32-wide d steps of S^T = K.Q^T
  constexpr int DB = D / 16;      // 16-wide d blocks of O^T
  constexpr int KB = KT / 16;     // 16-key blocks of S^T
  constexpr int KP = KT / 32;     // 32-key steps of O^T += V^T.P^T
  constexpr int PER = 2 * TL::NI / NW;   // DMA instructions per wave per stage
  // fragments read ahead per group: all of a tile's with one wavefront per
  // SIMD, half with more
  constexpr int KSPLIT = OCC > 1 ? 2 : 1;
  constexpr int VSPLIT = OCC > 1 ? 2 : 1;
  static_assert(STG >= 2 && STG <= 4, "ring depth");
  static_assert(PER * NW == 2 * TL::NI && PER % 2 == 0 && 2 * PER < 64, "DMA split");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // [stage][K tile | V tile]

  const auto &run = as_const(a.runs)[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, kg = lane >> 4;
  const int G = a.G, Hkv = a.Hkv, Hq = a.Hq;
  const int nt = run.tiles;                                  // the run's tiles, item after item
  const int64_t key_stride = int64_t(Hkv) * ROWB;            // bytes between keys

  // DMA instruction i of this wave covers tile block w + NW * (i % HPER) of
  // K (i < HPER) or V (i >= HPER); voff_lane is the lane's byte offset from
  // the tile's first key (tile row, swizzled source chunk)
  constexpr int HPER = PER / 2;
  int voff_lane[HPER];
#pragma unroll
  for (int i = 0; i < HPER; ++i) {
    const int row = (w + NW * i) * RPI + lane / CH;
    voff_lane[i] = int(row * key_stride + 16 * swz_chunk<D>(row, lane % CH));
  }
  const uint32_t lds0 = lds_addr(smem);

  // ---- DMA side: walks the run's tiles STG - 1 ahead of the compute side.
  // Per item: the tree's prefix of KV head g, and its rows.
  int d_item = run.first, d_tile = 0, d_end = 0, d_np = 0;
  const uint16_t *pk = nullptr, *pv = nullptr, *rk = nullptr, *rv = nullptr;
  uint32_t pre_bytes = 0, row_bytes = 0;
  auto d_enter = [&](int i) {
    const auto &e = as_const(a.items)[i];
    const int64_t head0 = int64_t(e.g) * D;
    d_item = i;
    d_tile = e.k0 / KT;
    d_end = e.k1 / KT;
    d_np = (e.kv_len + KT - 1) / KT;
    pre_bytes = e.kv_len > 0 ? uint32_t(int64_t(e.kv_len - 1) * key_stride + ROWB) : 0u;
    row_bytes = uint32_t(int64_t(e.tree_rows - 1) * key_stride + ROWB);
    pk = a.kv_k + e.kv_off * Hkv * D + head0;
    pv = a.kv_v + e.kv_off * Hkv * D + head0;
    rk = a.k_rot + int64_t(e.tree_start) * Hkv * D + head0;
    rv = a.v_rows + int64_t(e.tree_start) * Hkv * D + head0;
  };
  d_enter(run.first);
  auto issue = [&](int s) {                   // DMA the run's next tile into stage s % STG
    if (d_tile == d_end) d_enter(d_item + 1);
    const int t = d_tile++;
    const bool pre = t < d_np;
    const int vbase = int(int64_t((pre ? t : t - d_np) * KT) * key_stride);
    const i32x4 rsk = make_rsrc(pre ? pk : rk, pre ? pre_bytes : row_bytes);
    const i32x4 rsv = make_rsrc(pre ? pv : rv, pre ? pre_bytes : row_bytes);
    const uint32_t sbase = lds0 + uint32_t((s % STG) * 2 * TILEB) + uint32_t(w * 1024);
#pragma unroll
    for (int i = 0; i < HPER; ++i) dma16<kNtStream>(rsk, sbase + uint32_t(NW * i * 1024), vbase + voff_lane[i], 0);
#pragma unroll
    for (int i = 0; i < HPER; ++i) dma16<kNtStream>(rsv, sbase + uint32_t(TILEB + NW * i * 1024), vbase + voff_lane[i], 0);
  };

  // ---- compute side: the current item's query fragments (B operand of
  // S^T = K.Q^T, hi and lo), ancestor bits, prefix length and running
  // softmax state.  With D <= 128 an item's rows may come from several trees
  // of one pack (one KV segment): each query sees the first q_klen keys of
  // the prefix (its tree's length, kept in LDS for the masked tiles; c_kmin
  // is the item's smallest) and the pack's rows its ancestor bits (relative
  // to the pack's first row) select.  With D = 256 (no register to spare) a
  // pack is one tree and every query sees the item's c_kmin = kv_len keys.
  constexpr bool PACKS = D <= 128;
  __shared__ int q_klen[PACKS ? NW * 16 : 1];
  const int mq = w * 16 + n16;
  int c_item = run.first, c_tile = 0, c_end = 0, c_np = 0, c_kmin = 0, c_slot = 0;
  bool wave_on = false, qok = false;
  uint4 qh[DS], ql[DS];
  uint64_t anc = 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB];
  auto c_enter = [&](int i) {
    const auto &e = as_const(a.items)[i];
    c_item = i;
    c_tile = e.k0 / KT;
    c_end = e.k1 / KT;
    c_np = (e.kv_len + KT - 1) / KT;
    c_kmin = PACKS ? e.kv_min : e.kv_len;
    c_slot = e.slot;
    wave_on = w < (e.nq + 15) / 16;
    qok = wave_on && mq < e.nq;
    anc = 0;
    [[maybe_unused]] int klen = 0;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qh[ds] = ql[ds] = make_uint4(0, 0, 0, 0);
    if (qok) {
      const int m = e.m0 + mq;
      const int row = e.tree_start + m / G;
      const int head = e.g * G + m % G;
      const uint16_t *qp = a.q_rot + (int64_t(row) * Hq + head) * D + kg * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        qh[ds] = *reinterpret_cast<const uint4 *>(qp + ds * 32);
        ql[ds] = *reinterpret_cast<const uint4 *>(qp + a.q_lo_off + ds * 32);
      }
      anc = a.row_panc[row];
      if constexpr (PACKS) klen = a.row_klen[row];
    }
    // Complete these loads here: the compiler does not see the DMA, and
    // would otherwise re-wait for them (with every DMA in flight) inside the
    // tile loop.  Here the wait also covers the DMA already issued, which
    // the next tile needs anyway.
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      asm volatile("" : "+v"(qh[ds].x), "+v"(qh[ds].y), "+v"(qh[ds].z), "+v"(qh[ds].w));
      asm volatile("" : "+v"(ql[ds].x), "+v"(ql[ds].y), "+v"(ql[ds].z), "+v"(ql[ds].w));
    }
    asm volatile("" : "+v"(anc));
    if constexpr (PACKS) {
      asm volatile("" : "+v"(klen));
      if (kg == 0) q_klen[mq] = klen;   // read back by this wavefront only
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

#pragma unroll
  for (int s = 0; s < STG - 1; ++s)
    if (s < nt) issue(s);
  c_enter(run.first);

  for (int s = 0; s < nt; ++s) {
    const int ahead = min(STG - 2, nt - 1 - s);   // tiles in flight behind this one
    if (ahead >= 2)
      wait_and_barrier<2 * PER>();
    else if (ahead == 1)
      wait_and_barrier<PER>();
    else
      wait_and_barrier<0>();
    if (s + STG - 1 < nt) issue(s + STG - 1);
    if (wave_on) {
      const int t = c_tile;
      const uint8_t *kt_lds = smem + (s % STG) * 2 * TILEB;
      const uint8_t *vt_lds = kt_lds + TILEB;

      // S^T = K.(Q_hi + Q_lo)^T, KB blocks of 16 keys.  With one wavefront per
      // SIMD, every K and V^T fragment of the tile is read up front (their LDS
      // latency then overlaps the MFMAs and the softmax); with two, K and V^T
      // are read in halves.
      const int sl = lane & 15;
      const int ra0 = 4 * kg + (sl >> 2);       // V^T source row within a 32-key step
      auto read_k = [&](int ds, int kb) {
        const int row = 16 * kb + n16;
        return *reinterpret_cast<const uint4 *>(kt_lds + row * ROWB + 16 * swz_chunk<D>(row, ds * 4 + kg));
      };
      auto read_v = [&](int kp, int db) {
        const int ra = 32 * kp + ra0, rb = ra + 16;
        const int c = 2 * db + ((sl & 3) >> 1);
        const uint2 lo = lds_read_tr16(vt_lds + ra * ROWB + 8 * (sl & 1) + 16 * swz_chunk<D>(ra, c));
        const uint2 hi = lds_read_tr16(vt_lds + rb * ROWB + 8 * (sl & 1) + 16 * swz_chunk<D>(rb, c));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      f32x4 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      uint4 vf[KP][DB / VSPLIT];
#pragma unroll
      for (int part = 0; part < KSPLIT; ++part) {
        uint4 kf[DS / KSPLIT][KB];
#pragma unroll
        for (int dd = 0; dd < DS / KSPLIT; ++dd)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) kf[dd][kb] = read_k(part * (DS / KSPLIT) + dd, kb);
        if (part == 0) {
#pragma unroll
          for (int kp = 0; kp < KP; ++kp)
#pragma unroll
            for (int dd = 0; dd < DB / VSPLIT; ++dd) vf[kp][dd] = read_v(kp, dd);
        }
#pragma unroll
        for (int dd = 0; dd < DS / KSPLIT; ++dd)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int ds = part * (DS / KSPLIT) + dd;
            sacc[kb] = mfma16(kf[dd][kb], qh[ds], sacc[kb]);
            sacc[kb] = mfma16(kf[dd][kb], ql[ds], sacc[kb]);
          }
        // order: the K reads, then the S^T MFMAs with the V^T reads (two per
        // fragment) slotted one per MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, (DS / KSPLIT) * KB, 0);
        if (part == 0) {
#pragma unroll
          for (int m = 0; m < 2 * (DS / KSPLIT) * KB; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m < 2 * KP * (DB / VSPLIT)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * (DS / KSPLIT) * KB, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // visibility of the lane's 4 keys per block, as nibbles: a prefix tile
      // shows its first klen - key0 keys, a row tile the ancestor-or-self rows
      const bool pre = t < c_np;
      const int key0 = (pre ? t : t - c_np) * KT;
      const uint64_t rbits = (!pre && key0 < 64) ? (anc >> key0) : 0ull;
      const uint32_t rlo = uint32_t(rbits), rhi = uint32_t(rbits >> 32);
      float x[KB][4];
      float tmax = -INFINITY;
      if (pre && c_kmin - key0 >= KT) {
        // a prefix tile whose keys every query of the item sees (every
        // tile but the last prefix tiles and the row tiles): no mask.  Padding query lanes
        // (zero queries) get finite scores here that are never written out.
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[kb][i] = sacc[kb][i] * a.scale_log2;
            tmax = fmaxf(tmax, x[kb][i]);
          }
      } else {
        const int lim = pre ? (PACKS ? q_klen[mq] : c_kmin) - key0 : 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int vb = 16 * kb + 4 * kg;
          const uint32_t nib_pre = (1u << min(max(lim - vb, 0), 4)) - 1u;
          uint32_t nib_row = 0;
          if (16 * kb < 64) nib_row = ((kb < 2 ? rlo : rhi) >> ((16 * kb & 31) + 4 * kg)) & 15u;
          const uint32_t nib = qok ? (pre ? nib_pre : nib_row) : 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[kb][i] = ((nib >> i) & 1u) ? sacc[kb][i] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[kb][i]);
          }
        }
      }
      // Online softmax (log2 domain) with a lazy reference: the reference m_run
      // moves only when the tile max exceeds it by more than 8, so p <= 2^8 and
      // the rescale of O is usually skipped.  l_run is the lane's own share.
      tmax = rows4_max(tmax);
      const bool up = tmax > m_run + 8.f;
      const float alpha = up ? exp2f(m_run - tmax) : 1.f;
      m_run = up ? tmax : m_run;
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[kb][i] = exp2f(x[kb][i] - m_use);
          ls += x[kb][i];
        }
      l_run = l_run * alpha + ls;
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = o[db] * alpha;
      }
      // O^T += V^T.(P_hi + P_lo)^T per 32 keys.  Operand slot 8*kg + t holds
      // key 4*kg + t (t < 4) or 16 + 4*kg + t - 4 (t >= 4) of the 32, on both
      // operands.  V^T fragments come from transposing reads: source lane s of
      // the 16-lane group addresses tile row r0 + (s >> 2), columns
      // 16*db + 4*(s & 3) .. +3.
#pragma unroll
      for (int kp = 0; kp < KP; ++kp) {
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2)
          split_bf2(x[2 * kp + (t2 >> 1)][2 * (t2 & 1)], x[2 * kp + (t2 >> 1)][2 * (t2 & 1) + 1], ph[t2], pl[t2]);
        const uint4 pfh = make_uint4(ph[0], ph[1], ph[2], ph[3]);
        const uint4 pfl = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
        for (int part = 0; part < VSPLIT; ++part) {
          if (part > 0) {
#pragma unroll
            for (int dd = 0; dd < DB / VSPLIT; ++dd) vf[kp][dd] = read_v(kp, part * (DB / VSPLIT) + dd);
          }
#pragma unroll
          for (int dd = 0; dd < DB / VSPLIT; ++dd) {
            const int db = part * (DB / VSPLIT) + dd;
            o[db] = mfma16(vf[kp][dd], pfh, o[db]);
            o[db] = mfma16(vf[kp][dd], pfl, o[db]);
          }
        }
      }
    }

    // ---- the item ends with this tile: its partial results, then the next
    // item's queries
    if (++c_tile == c_end) {
      const float l_all = rows4_sum(l_run);
      if (qok) {
        const int64_t slot = int64_t(c_slot) + mq;
        if (kg == 0) {
          a.part_ml[2 * slot] = m_run;
          a.part_ml[2 * slot + 1] = l_all;
        }
        float *po = a.part_o + slot * D + 4 * kg;
        if constexpr (NTP) {
#pragma unroll
          for (int db = 0; db < DB; ++db) __builtin_nontemporal_store(o[db], reinterpret_cast<f32x4 *>(po + db * 16));
        } else {
#pragma unroll
          for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4 *>(po + db * 16) = o[db];
        }
      }
      if (s + 1 < nt) c_enter(c_item + 1);
    }
  }
}

// Combine the partial records of one (row, query head) and write o in the
// projection's activation format.  WPP wavefronts per (row, query head): one
// when its query group has few items (four pairs per workgroup), four when
// it has many (the items split round robin, the four sums added in LDS).
// Lane c owns elements [c E, c E + E) of o, E = D / 64.  Each wavefront
// reads the (max, sum) records once (each lane folds its share into a
// running pair) and leaves the item weights exp2(m_t - M) in its own LDS
// row; then it sums the o records, four in flight.
template <int D, int WPP>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a, int n_pairs) {
  constexpr int E = D / 64;
  typedef float fvec __attribute__((ext_vector_type(E)));
  __shared__ float wl[4][kMaxSplits];
  __shared__ fvec red[WPP > 1 ? WPP : 1][64];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), c = threadIdx.x & 63;
  const int pair = WPP > 1 ? int(blockIdx.x) : int(blockIdx.x) * 4 + w;
  if (WPP == 1 && pair >= n_pairs) return;    // no workgroup-wide synchronisation with one wave per pair
  const int i = pair / a.Hq, h = pair % a.Hq;
  const int G = a.Hq / a.Hkv;
  const int r = as_const(a.row_tree)[i], loc = as_const(a.row_local)[i];
  const int g = h / G, m = loc * G + h % G;
  const int qg = m / kItemQ, mi = m % kItemQ;
  const auto &gr = as_const(a.groups)[(r * a.Hkv + g) * a.qg_max + qg];
  const int cnt = min(gr.count, kMaxSplits);   // the plan keeps it <= kMaxSplits
  const int64_t base = int64_t(gr.slot) + mi, stride = gr.nq;

  // (max, sum) over the items; an item that saw no key of this query has
  // max -inf and sum 0
  float Mi = -INFINITY, Li = 0.f;
  for (int t = c; t < cnt; t += 64) {
    const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + 2 * (base + t * stride));
    wl[w][t] = ml.x;
    if (ml.x == -INFINITY) continue;
    if (ml.x > Mi) {
      Li = (Mi == -INFINITY ? 0.f : Li * exp2f(Mi - ml.x)) + ml.y;
      Mi = ml.x;
    } else {
      Li += ml.y * exp2f(ml.x - Mi);
    }
  }
  const float M = wave_max_dpp(Mi);
  const float L = wave_sum_dpp(Mi == -INFINITY ? 0.f : Li * exp2f(Mi - M));
  for (int t = c; t < cnt; t += 64) {         // the lane's own entries: no other lane writes them
    const float mt = wl[w][t];
    wl[w][t] = mt == -INFINITY ? 0.f : exp2f(mt - M);
  }
  // the wavefront's LDS writes above precede its reads below in LDS order

  auto orec = [&](int t) { return *reinterpret_cast<const fvec *>(a.part_o + (base + t * stride) * D + c * E); };
  fvec acc0 = fvec(0.f), acc1 = fvec(0.f), acc2 = fvec(0.f), acc3 = fvec(0.f);
  const int t0 = WPP > 1 ? w : 0;
  int t = t0;
  for (; t + 3 * WPP < cnt; t += 4 * WPP) {
    const fvec o0 = orec(t), o1 = orec(t + WPP), o2 = orec(t + 2 * WPP), o3 = orec(t + 3 * WPP);
    acc0 += wl[w][t] * o0;
    acc1 += wl[w][t + WPP] * o1;
    acc2 += wl[w][t + 2 * WPP] * o2;
    acc3 += wl[w][t + 3 * WPP] * o3;
  }
  for (; t < cnt; t += WPP) acc0 += wl[w][t] * orec(t);
  fvec val = (acc0 + acc1) + (acc2 + acc3);
  if constexpr (WPP > 1) {
    red[w][c] = val;
    __syncthreads();
    val = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
  }
  // The keys rotated in this step (the row's ancestors and itself) reached
  // the attention tiles rounded to bf16.  Each contributed 2^(x~ - M) v to
  // val and 2^(x~ - M) to L, x~ the log2-scaled score against the rounded key;
  // swap in 2^(x - M), x the score against the key's hi + lo pair (about 16
  // bits).  x~ is recomputed in fp32 from the same bf16 operands the tiles
  // multiplied.  Lane c holds elements [c E, c E + E) of the query and keys.
  float Lx = L;
  if (a.row_anc) {
    const int64_t qoff = (int64_t(i) * a.Hq + h) * D + c * E;
    float qv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] = bf2f(a.q_rot[qoff + e]) + bf2f(a.q_rot[a.q_lo_off + qoff + e]);
    const int ts = as_const(a.tree_start)[as_const(a.row_tree_real)[i]];
    uint64_t bits = a.row_anc[i];
    // WPP > 1: wavefront w takes the keys w, w + WPP, ... (in bit order) and
    // its sums are added in wavefront order below; the LDS records of the
    // merge above are no longer read, so they take these sums
    fvec dv = fvec(0.f);
    float dl = 0.f;
    for (int k = 0; bits; ++k) {
      const int j = __builtin_ctzll(bits);
      bits &= bits - 1;
      if (WPP > 1 && k % WPP != w) continue;
      const int64_t koff = (int64_t(ts + j) * a.Hkv + g) * D + c * E;
      float st = 0.f, sx = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float kh = bf2f(a.k_rot[koff + e]), kl = bf2f(a.k_rot[a.k_lo_off + koff + e]);
        st = fmaf(kh, qv[e], st);
        sx = fmaf(kh + kl, qv[e], sx);
      }
      st = wave_sum_dpp(st);
      sx = wave_sum_dpp(sx);
      const float dp = exp2f(sx * a.scale_log2 - M) - exp2f(st * a.scale_log2 - M);
      dl += dp;
#pragma unroll
      for (int e = 0; e < E; ++e) dv[e] = fmaf(dp, bf2f(a.v_rows[koff + e]), dv[e]);
    }
    if constexpr (WPP > 1) {
      __shared__ float dls[WPP];
      __syncthreads();   // every wavefront has read the merge records
      red[w][c] = dv;
      if (c == 0) dls[w] = dl;
      __syncthreads();
      if (w != 0) return;
      dv = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
      dl = (dls[0] + dls[1]) + (dls[2] + dls[3]);
    }
    Lx += dl;
    val += dv;
  } else if constexpr (WPP > 1) {
    if (w != 0) return;
  }
  val = val / Lx;

  const int64_t idx = int64_t(i) * a.Hq * D + int64_t(h) * D + c * E;
  uint16_t hi[E], lo[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (a.mode == ACT_SPLIT || a.mode == ACT_SPLIT_BLOCKED)
      split_h(val[e], hi[e], lo[e]);
    else
      hi[e] = f2h(val[e]);
  }
  if (a.mode == ACT_F16_BLOCKED || a.mode == ACT_SPLIT_BLOCKED) {
    // blocked fp16 layout of the tiled W_o launch (K = Hq * D); the lane's E
    // elements share one 16-B chunk; the lo plane (ACT_SPLIT_BLOCKED) in the
    // same layout lo_off elements on
    const int k = h * D + c * E, R = i & 255, q = (k >> 3) & 3;
    const int64_t b = (int64_t(i >> 8) * ((a.Hq * D) >> 5) + (k >> 5)) * 8192;
    uint16_t *dst = a.out + b + R * 32 + (blk_slot(q, R) << 3) + (k & 7);
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = hi[e];
    if (a.mode == ACT_SPLIT_BLOCKED) {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[a.lo_off + e] = lo[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) a.out[idx + e] = hi[e];
    if (a.mode == ACT_SPLIT) {
#pragma unroll
      for (int e = 0; e < E; ++e) a.out[a.lo_off + idx + e] = lo[e];
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 attention: one workgroup per (row, query head), keys in tiles of 256.
// ----------------------------------------------------------------------------

__device__ __forceinline__ float block_max256(float v, float *red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
  __shared__ float q_s[256];
  __shared__ float p_s[256];
  __shared__ float red[4];
  const int i = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int D = a.D, tid = threadIdx.x;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int r = a.row_tree[i];
  const int s0 = a.tree_start[r], T = a.tree_rows[r], klen = a.tree_kv_len[r];
  const int64_t koff = a.tree_kv_off[r];
  const uint64_t anc = a.row_anc[i];
  const int nk = klen + T;
  if (tid < D) q_s[tid] = a.q_rot[(int64_t(i) * a.Hq + h) * D + tid];
  __syncthreads();
  auto kptr = [&](int v, const float *pre, const float *rows) -> const float * {
    return v < klen ? pre + ((koff + v) * a.Hkv + g) * int64_t(D)
                    : rows + (int64_t(s0 + v - klen) * a.Hkv + g) * D;
  };
  const float scale = 1.0f / sqrtf(float(D));
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int kt = 0; kt < nk; kt += 256) {
    const int v = kt + tid;
    float x = -INFINITY;
    if (v < nk && (v < klen || ((anc >> (v - klen)) & 1ull))) {
      const float *kp = kptr(v, a.kv_k, a.k_rot);
      float s = 0.f;
      for (int c = 0; c < D; ++c) s = fmaf(q_s[c], kp[c], s);
      x = s * scale;
    }
    const float tmax = block_max256(x, red);
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_ref);
    const float p = expf(x - m_ref);
    p_s[tid] = p;
    const float rs = block_sum256(p, red);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (tid < D) {
      acc *= alpha;
      const int lim = min(256, nk - kt);
      for (int j = 0; j < lim; ++j) {
        const float pj = p_s[j];
        if (pj != 0.f) acc = fmaf(pj, kptr(kt + j, a.kv_v, a.v_rows)[tid], acc);
      }
    }
    __syncthreads();
  }
  if (tid < D) a.out[int64_t(i) * a.Hq * D + int64_t(h) * D + tid] = acc / l_run;
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

void launch_rope_f32(const float *q, const float *k, float *qo, float *ko, const int32_t *row_pos, int n, int Hq,
                     int Hkv, int D, double base, hipStream_t s) {
  const dim3 grid(n, (Hq + Hkv) * (D / 2) / 256 + ((Hq + Hkv) * (D / 2) % 256 != 0));
  hipLaunchKernelGGL(rope_rows_kernel<float>, grid, dim3(256), 0, s, q, k, qo, ko, row_pos, Hq, Hkv, D, base);
}

template <int D, int NW, int STG, int OCC, bool NTP>
static void launch_attn_ddn(const AttnArgs &a, int n_runs, hipStream_t s) {
  constexpr size_t lds = attn_lds_bytes<D, STG>();
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(attn_mfma_kernel<D, NW, STG, OCC, NTP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  hipLaunchKernelGGL((attn_mfma_kernel<D, NW, STG, OCC, NTP>), dim3(n_runs), dim3(64 * NW), lds, s, a);
}

template <int D, int NW, int STG, int OCC>
static void launch_attn_dd(const AttnArgs &a, int n_runs, hipStream_t s) {
  if (a.nt_part)
    launch_attn_ddn<D, NW, STG, OCC, true>(a, n_runs, s);
  else
    launch_attn_ddn<D, NW, STG, OCC, false>(a, n_runs, s);
}

// Four wavefronts (up to 64 query vectors): a 2-stage ring (64 KB of LDS)
// so that two workgroups share a compute unit and hide each other's
// latencies.  Eight wavefronts: a 4-stage ring, one workgroup per unit.
void launch_attn_mfma(const AttnArgs &a, int n_runs, int D, int max_qblocks, hipStream_t s) {
  const bool eight = max_qblocks > 4;
  if (D == 64) eight ? launch_attn_dd<64, 8, 4, 2>(a, n_runs, s) : launch_attn_dd<64, 4, 2, 2>(a, n_runs, s);
  if (D == 128) eight ? launch_attn_dd<128, 8, 4, 2>(a, n_runs, s) : launch_attn_dd<128, 4, 2, 2>(a, n_runs, s);
  if (D == 256) eight ? launch_attn_dd<256, 8, 4, 2>(a, n_runs, s) : launch_attn_dd<256, 4, 2, 2>(a, n_runs, s);
}

template <int D>
static void launch_merge_d(const MergeArgs &a, int pairs, bool many, hipStream_t s) {
  if (many)
    hipLaunchKernelGGL((attn_merge_kernel<D, 4>), dim3(pairs), dim3(256), 0, s, a, pairs);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, 1>), dim3((pairs + 3) / 4), dim3(256), 0, s, a, pairs);
}

// Four wavefronts per (row, query head) once query groups average 16 items
// or more.
void launch_attn_merge(const MergeArgs &a, int n_rows, int D, double mean_items, hipStream_t s) {
  const int pairs = n_rows * a.Hq;
  const bool many = mean_items >= 16.0;
  if (D == 64) launch_merge_d<64>(a, pairs, many, s);
  if (D == 128) launch_merge_d<128>(a, pairs, many, s);
  if (D == 256) launch_merge_d<256>(a, pairs, many, s);
}

void launch_attn_f32(const AttnF32Args &a, int n_rows, hipStream_t s) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(n_rows * a.Hq), dim3(256), 0, s, a);
}

}  // namespace sv
