// Commit of a verify step: each tree's accepted path joins its KV cache
// right after the visible prefix (sionic.ai "Solar Open2 250B DSpark",
// section 1: generation resumes after the matching leading drafts; section
// 6: committing accepted tokens is the step that follows verify).  The path
// is the root, then every accepted draft in depth order, ending at the
// tree's last accepted row; its K rows are the keys the verify step rotated
// at their semantic positions, its V rows the row values.  The bonus token
// is not written: it is the next step's root.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "plan.hpp"

namespace sv {

// One workgroup per tree: the tree's parent map goes to LDS, one thread
// walks up from the last accepted row, then all threads copy the path rows
// (16 B per thread step, K and V).
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
  __shared__ int32_t par[kMaxTreeRows];
  __shared__ int32_t path[kMaxTreeRows];
  __shared__ int32_t n_path;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int s0 = a.tree_start[t], rows = a.tree_rows[t];
  for (int i = tid; i < rows; i += 256) par[i] = a.row_parent[s0 + i] - s0;   // roots: -1 - s0 < 0
  __syncthreads();
  if (tid == 0) {
    const int acc = a.accept_len[t];
    int cur = a.last_row[t] - s0;
    int d = acc - 1;
    if (acc < 1 || acc > rows) d = -2;   // not a result of this tree: copy nothing
    // depth of last_row must be acc - 1 (d stays in [0, rows))
    while (d >= 0 && cur >= 0 && cur < rows) {
      path[d] = cur;
      cur = par[cur];
      --d;
    }
    // a consistent run ends the walk exactly at the root
    n_path = (d == -1 && cur < 0) ? acc : 0;
  }
  __syncthreads();
  const int np = n_path;
  const int chunks = a.row_bytes / 16;
  const int64_t base = a.kv_off[t] + a.kv_len[t];
  for (int x = tid; x < np * chunks; x += 256) {
    const int j = x / chunks, c = x % chunks;
    const int64_t src = int64_t(s0 + path[j]) * a.row_bytes + c * 16;
    const int64_t dst = (base + j) * a.row_bytes + c * 16;
    *reinterpret_cast<uint4 *>(a.kv_k + dst) = *reinterpret_cast<const uint4 *>(a.k_rot + src);
    *reinterpret_cast<uint4 *>(a.kv_v + dst) = *reinterpret_cast<const uint4 *>(a.v_rows + src);
  }
}

void launch_commit(const CommitArgs &a, int n_roots, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(n_roots), dim3(256), 0, s, a);
}

}  // namespace sv
