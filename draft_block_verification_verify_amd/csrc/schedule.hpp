// Verify budget over a batch of requests (host only, no HIP): which draft
// candidates each request verifies in the next step.  See
// spec_verify_schedule in spec_verify.h.
#pragma once

#include <cstdint>
#include <string>

namespace sv {

// Step time of a batch of `rows` rows on the measured curve: linear between
// points, the first value below the first point, extended from the last two
// points past the last one.
double curve_step_ms(int n_curve, const int32_t *curve_rows, const float *curve_ms, double rows);

// Returns 0 (P_OK) or a PlanStatus code with *err set.  On success writes
// selected[] (0/1 per candidate), the expected tokens and the step time.
int schedule_budget(int n_req, const int32_t *n_cand, const int32_t *cand_parent, const float *cand_conf,
                    int n_curve, const int32_t *curve_rows, const float *curve_ms, int max_rows,
                    int32_t *selected, double *expected_tokens, double *step_ms, std::string *err);

}  // namespace sv
