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

// Launch plan of a prefill of `batch` sequences of L tokens.
//
// Forward: the main scan runs `chunks` chunks of chunk_len tokens per
// sequence.  With chunks > 1, pass 1 scans every chunk from a zero state
// (chunk 0 from h0), a combine folds the chunks' (decay, end state) pairs into
// each chunk's true starting state, and pass 2 rescans each later chunk from
// it only until the carried-in part of the state has decayed below fp32
// resolution.
//
// Backward: its sweeps run one wave per (sub-chunk, 64 channels), sub-chunks
// of sub_len tokens (subs per sequence).  Pass 1 records the chunk-local
// state at every sub-chunk boundary it passes, so the backward can take its
// starting states from a prefill's workspace.  With chunks == subs == 1
// nothing is recorded and the prefill is one plain sweep.
struct Plan {
  int chunks;              // forward chunks per sequence
  int64_t chunk_len;       // tokens per forward chunk (a multiple of kTok)
  int subs;                // sub-chunks per sequence (the backward's chunks)
  int64_t sub_len;         // tokens per sub-chunk (a multiple of kTok)
  bool recorded() const { return chunks > 1 || subs > 1; }
};

Plan choose_plan(int64_t batch, int64_t L, int64_t d_inner);
double wave_efficiency(double waves);

size_t round_up(size_t v);
// Workgroups of 256 for a grid-stride pass over n elements (capped).
unsigned copy_grid(int64_t n);
// Bytes of the RMSNorm region of a prefill workspace for `rows` token rows.
size_t rms_bytes(int64_t rows);
// Workspace of a recording prefill, in this order: a tag (first, so that its
// place does not depend on the plan), each forward chunk's end record (its
// chunk-local end state [b][chunks][16][d] and delta sum [b][chunks][d]), a
// per-(chunk, channel) flag of negative time steps, per (chunk, 64-channel
// group) the first token pass 1 wrote y for, the true starting states
// of the forward chunks [b][chunks][16][d] (chunk 0: unused), and the
// sub-chunk records (chunk-local state at the end of sub-chunk s
// [b][subs][16][d] and the delta sum from its chunk's start [b][subs][d];
// the last sub-chunk has none).  The fields are region sizes; the off_*
// functions give byte offsets.
struct WsLayout {
  size_t tag, eS, eL, neg, from, H, sS, sL, total;
  size_t off_eS() const { return tag; }
  size_t off_eL() const { return off_eS() + eS; }
  size_t off_neg() const { return off_eL() + eL; }
  size_t off_from() const { return off_neg() + neg; }
  size_t off_H() const { return off_from() + from; }
  size_t off_sS() const { return off_H() + H; }
  size_t off_sL() const { return off_sS() + sS; }
};
WsLayout ws_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p);

// The tag a recording prefill writes at the start of its workspace: what
// produced the states there.  The backward that reuses them compares it with
// its own sizes and plan on the GPU.  variant: 0 for the plain recurrence,
// else 1 (conv) | 2 (softplus) | 4 (trapezoidal) | 8 (RMSNorm).
constexpr int kTagWords = 8;
constexpr int64_t kTagMagic = 0x6a7363616e746167LL;
struct Tag { int64_t w[kTagWords]; };
Tag make_tag(int64_t batch, int64_t L, int64_t d_inner, const Plan& p, int variant);

// The records the backward derives its sub-chunk starting states from (plan
// p with p.subs > 1): the chunk-local state and delta sum at every sub-chunk
// boundary, sS[b][s][n][d] and sL[b][s][d] (boundary s + 1 of sequence b),
// and the true starting state of every forward chunk, H[b][c][n][d].  With
// `saved` (a plain prefill's workspace, as jscan_prefill leaves it) they are
// there already; otherwise a state-only pass and the combine write them into
// `rec` (ws_layout(...).total bytes).
struct SubRecords {
  const float* sS;
  const float* sL;
  const float* H;
};
jscan_status backward_records(jscan_io io, int64_t batch, int64_t L, int64_t d_inner, const void* x,
                              const void* delta, const float* A, const void* B, const float* h0, char* rec,
                              const char* saved, const Plan& p, hipStream_t st, SubRecords* out);

}  // namespace jscan_detail
