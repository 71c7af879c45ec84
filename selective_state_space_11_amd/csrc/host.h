// Host-side pieces of libjscan shared by the forward and backward entry
// points: error reporting, argument checks, the launch plan and the
// workspace layout of chunked plans.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "jscan.h"

namespace jscan_detail {

// Text of the last error on this thread (jscan_last_error).
extern thread_local std::string t_last_error;

jscan_status fail(jscan_status s, const std::string& msg);
jscan_status hip_fail(hipError_t e, const char* what);
bool mul_ok(int64_t a, int64_t b, int64_t* out);

struct Range { const void* p; size_t bytes; const char* name; };

bool overlap(const Range& a, const Range& b);
bool aligned16(const void* p);
jscan_status check_common(int64_t d_state, jscan_io io);
// Every output against every input and every other output.  An output may be
// the very same buffer as one input (`same_ok`, e.g. an in-place state carry).
jscan_status check_ranges(const Range* in, int n_in, const Range* out, int n_out, const void* same_ok = nullptr);
bool sizes_ok(int64_t batch, int64_t L, int64_t d_inner);

// Launch plan.  The main scan runs `chunks` chunks of chunk_len tokens per
// sequence with K waves per 64 channels.  When chunks > 1, the tokens before
// the last chunk are cut into segments of seg_len tokens (seg_per_chunk per
// chunk) for the chunk-local pass, so that pass fills the GPU on its own.
struct Plan {
  int K;
  int chunks;
  int64_t chunk_len;
  int seg_per_chunk;
  int64_t seg_len;
  int64_t segments() const { return chunks > 1 ? (int64_t)(chunks - 1) * seg_per_chunk : 0; }
};

Plan choose_plan(int64_t batch, int64_t L, int64_t d_inner);
Plan make_plan(int64_t batch, int64_t L, int64_t d_inner, int K, int64_t C_target);
double wave_efficiency(double waves);

size_t round_up(size_t v);
// Workspace of a chunked prefill plan, in this order: a tag (first, so that
// its place does not depend on the plan), chunk-local end states, delta sums,
// chunk starting states (all state-major) and a conv-history copy.  The
// fields are region sizes; the off_* functions give byte offsets.
struct WsLayout {
  size_t tag, S, dsum, hstart, hist, total;
  size_t off_S() const { return tag; }
  size_t off_dsum() const { return tag + S; }
  size_t off_hstart() const { return tag + S + dsum; }
  size_t off_hist() const { return tag + S + dsum + hstart; }
};
WsLayout ws_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p);

// The tag a chunked prefill writes at the start of its workspace: what produced
// the chunk starting states there.  The backward that reuses them compares it
// with its own sizes and plan on the GPU.  variant: 0 for the plain
// recurrence, else 1 (conv) | 2 (softplus) | 4 (trapezoidal) | 8 (RMSNorm).
constexpr int kTagWords = 8;
constexpr int64_t kTagMagic = 0x6a7363616e746167LL;
struct Tag { int64_t w[kTagWords]; };
Tag make_tag(int64_t batch, int64_t L, int64_t d_inner, const Plan& p, int variant);

// Launches the chunk-local pass and the combine of plan p (chunks > 1):
// afterwards ws holds, at ws_layout's off_hstart(), hstart[b][c][n][d] = the
// state before chunk c's first token (c = 0: h0 or zero).
jscan_status forward_chunk_starts(jscan_io io, int64_t batch, int64_t L, int64_t d_inner, const void* x,
                                  const void* delta, const float* A, const void* B, const float* h0, char* ws,
                                  const Plan& p, hipStream_t st);

}  // namespace jscan_detail
