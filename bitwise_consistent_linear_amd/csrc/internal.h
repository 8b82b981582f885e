// Declarations shared by the library's own sources (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "gdn_cpr.h"

#define GDN_EXPORT __attribute__((visibility("default")))

namespace gdn {

// Thread-local error text behind gdn_last_error().
gdn_status_t fail(gdn_status_t status, const std::string &message);
gdn_status_t ok();

void sha256(const uint8_t *msg, size_t len, uint8_t out[32]);
bool admitted_chunk(int32_t chunk);
bool admitted_dk(int32_t d_k);
std::string contract_text(int32_t chunk, int32_t d_k);

enum ScanMode : int32_t { kTrainer = 0, kPrefill = 1 };

// Arguments of one scan launch (trainer_fwd or prefill); validated on the host.
struct ScanArgs {
  int32_t num_seqs, num_qk_heads, num_v_heads, d_k, d_v, chunk;
  int32_t bf16;
  int32_t mode;
  int64_t total_tokens;
  int64_t total_chunks;
  const int32_t *cu_seqlens;
  const void *q, *k, *v;
  const float *a, *b, *initial_state;
  float *o, *chunk_states, *final_state;
};

// Arguments of one decode-step launch; validated on the host.
struct DecodeArgs {
  int32_t num_seqs, num_qk_heads, num_v_heads, d_k, d_v, chunk;
  int32_t bf16;
  const int32_t *pos;
  const void *q, *k, *v;
  const float *a, *b;
  float *state, *o, *resync_states;
};

// Arguments of the backward (plan, state, chunk and combine kernels); validated on the host.
struct BwdArgs {
  int32_t num_seqs, num_qk_heads, num_v_heads, d_k, d_v, chunk;
  int32_t bf16;
  int32_t slots_max;   // chunk slots the plan may fill: total_chunks + num_seqs
  int32_t row_blocks;  // blocks of 32 rows per value head in the chunk kernel
  int32_t whole;       // set by the launcher: the branch-free chunk kernel runs after the
                       // general one, which then takes only chunks with a partial sub-block
  int64_t total_tokens;
  int64_t total_chunks;
  const int32_t *cu_seqlens;
  const void *q, *k, *v;
  const float *a, *b, *initial_state, *chunk_states, *d_o, *d_final_state;
  float *dq, *dk, *dv, *da, *db, *d_initial_state;
  // workspace
  int32_t *plan;        // [0]: slots used; then (sequence, chunk) pairs
  int32_t *plan_cbase;  // [N]: index of each sequence's first chunk state
  float *dsh_bnd;       // [total_chunks, Hv, d_v, d_k]: dL/ds at chunk ends
  float *partials;      // [T, Hv, row_blocks, 2 d_k + 4]: row-block sums of the shares
                        // (dq, dk, da, db, two padding slots: rows of whole float4)
};

// Byte offsets of the backward workspace's parts (each 256-byte aligned).
struct BwdWorkspace {
  int64_t plan_off, plan_bytes, cbase_off, cbase_bytes, dsh_off, dsh_bytes;
  int64_t partials_off, partials_bytes, total, slots_max;
};

// Bytes of the fixed device array behind gdn_cpr_trainer_bwd_noalloc, and its address on
// the current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = GDN_CPR_BWD_NOALLOC_MAX_BYTES;
hipError_t noalloc_scratch(void **ptr);

int backward_row_blocks(int d_v);
BwdWorkspace backward_workspace(int64_t num_seqs, int64_t num_v_heads, int64_t d_k,
                                int64_t d_v, int64_t total_tokens, int64_t total_chunks);
int64_t backward_state_grid(const BwdArgs &args, int lanes_per_row);
// seq: one chunk-pass workgroup per (sequence, value head, row block), sweeping the
// sequence's chunks in reverse (no state pass); else one per (chunk, value head, row block).
int64_t backward_chunk_grid(const BwdArgs &args, bool seq);
hipError_t launch_backward(const BwdArgs &args, int lanes_per_row, bool seq, hipStream_t stream);

// Arguments of the two-level CPR kernels (scan: trainer / prefill; or one decode step);
// validated on the host.
struct Cpr2Args {
  int32_t num_seqs, num_qk_heads, num_v_heads, d_k, d_v, chunk;
  int32_t bf16;
  int32_t decode;     // 1: one decode step (tokens from the cache), 0: a packed batch
  int32_t slots_max;  // chunk slots the plan may fill: total_chunks + num_seqs
  int64_t total_tokens, total_chunks;
  const int32_t *cu_seqlens, *pos;
  const void *q, *k, *v;
  const float *a, *b, *initial_state;
  float *o, *chunk_states, *final_state;  // chunk_states: S after each full chunk
  float *trans_a, *trans_b;               // A_c [.., Hv, d_k, d_k], B_c [.., Hv, d_v, d_k]
  float *state, *boundary, *resync;       // decode
  void *cache_k, *cache_v;                // decode: [N * C, Hk, d_k], [N * C, Hv, d_v]
  float *cache_a, *cache_b;               // decode: [N * C, Hv]
  int32_t *plan, *plan_cbase;
};
bool cpr2_dk_admitted(int d_k);
// Byte offsets of a two-level workspace: the plan and chunk bases (batch only), A_c, B_c
// (one per full chunk; decode: one per sequence) and, for prefill, the boundary states.
struct Cpr2Layout {
  int64_t plan_off, cbase_off, ta_off, tb_off, cs_off, total;
};
Cpr2Layout cpr2_layout(int64_t num_seqs, int64_t num_v_heads, int64_t d_k, int64_t d_v,
                       int64_t total_chunks, bool decode, bool need_states);
int64_t cpr2_max_grid(const Cpr2Args &args);
hipError_t launch_cpr2_scan(const Cpr2Args &args, hipStream_t stream);
hipError_t launch_cpr2_decode_tail(const Cpr2Args &args, const void *k, const void *v,
                                   const float *a, const float *b, hipStream_t stream);
std::string cpr2_contract_text(int32_t chunk, int32_t d_k);

// Arguments of one linear-region launch (Y = X W); validated on the host.
struct LinearArgs {
  int64_t m, n;
  int32_t k;
  int32_t x_bf16, w_bf16;
  const void *x, *w;
  float *y;
};
bool linear_k_admitted(int64_t k);
int64_t linear_grid(const LinearArgs &args);
hipError_t launch_linear(const LinearArgs &args, hipStream_t stream);

// Enqueue the kernels. lanes_per_row is 16, 8 or 4; a scan workgroup has 256 threads, or
// 512 with 16 lanes per row and 64-token stages; each group of lanes_per_row lanes holds one
// row, or two (rows_per_group = 2, at 4 lanes per row in 256-thread workgroups with
// 16-token stages). Return the HIP launch status.
hipError_t launch_scan(const ScanArgs &args, int lanes_per_row, int stage_tokens, int threads,
                       int rows_per_group, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &args, int lanes_per_row, hipStream_t stream);

// Number of workgroups a scan or decode launch uses (for the host-side size claims).
int64_t scan_grid(const ScanArgs &args, int lanes_per_row, int threads, int rows_per_group);
int64_t decode_grid(const DecodeArgs &args, int lanes_per_row);

}  // namespace gdn
