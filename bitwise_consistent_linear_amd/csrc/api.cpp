// C ABI entry points: host-side claims, identity check, dispatch to the HIP kernels.
//
// Every argument claim is checked here, before anything is enqueued, so that a refused
// call leaves all buffers untouched. IsoExec checks its claims and identities at run time
// (IsoExec, aihirek.info, section on the contract and common model; agentlenshq.com,
// section on contract structure: claims and identities).

#include <algorithm>
#include <array>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace gdn {
namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxInt32 = 2147483647;
// Elements of one token across all value heads (Hv * max(d_k, d_v)): bounded so that the
// kernels' offsets inside a stage of tokens fit in 32 bits.
constexpr int64_t kMaxHeadWidth = int64_t(1) << 20;

bool aligned(const void *p, size_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

// Lanes per state row: GDN_CPR_LANES_PER_ROW overrides the automatic choice.
int lanes_override() {
  const char *env = std::getenv("GDN_CPR_LANES_PER_ROW");
  if (env && *env) {
    const int v = std::atoi(env);
    if (v == 16 || v == 8 || v == 4) return v;
  }
  return 0;
}

// SIMDs of the current device (4 per compute unit), read once per device.
int64_t device_simds() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    v = 4 * cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Scan: the fewer the rows, the more lanes per row. A row on 16 lanes needs the most
// instructions but gives 4x the waves of 4 lanes per row; the recurrence is serial along
// the tokens, so with at most one wave per SIMD latency dominates and more lanes win, while
// with many waves per SIMD issue dominates and fewer lanes (fewer reduction steps) win.
// At two waves per SIMD, 16 lanes per row beat one wave of 8 (measured on the 8192-row
// trainer workload: the second wave issues its LDS and scalar work beside the first's
// vector work, which a lone wave cannot).
int scan_lanes(const ScanArgs &a) {
  if (const int o = lanes_override()) return o;
  const int64_t rows = (int64_t)a.num_seqs * a.num_v_heads * a.d_v;
  const int64_t simds = device_simds();
  if (rows / 4 <= 2 * simds) return 16;  // <= 2 waves per SIMD with 16 lanes per row
  if (rows / 8 <= simds) return 8;       // <= 1 wave per SIMD with 8 lanes per row
  return 4;
}

// Threads per scan workgroup: 512 (32 rows at 16 lanes per row) where two waves per SIMD
// run at 16 lanes per row with bf16 inputs, d_v a multiple of 32 and, for the trainer,
// C >= 64: one workgroup per CU then stages 64 tokens once for both waves of every SIMD,
// where two 256-thread workgroups would each stage 32. 256 otherwise.
// GDN_CPR_SCAN_THREADS=256 keeps 256; =512 takes 512 wherever it is admitted, whatever the
// number of rows (the same bits either way).
int scan_threads(const ScanArgs &a, int L) {
  const char *env = std::getenv("GDN_CPR_SCAN_THREADS");
  if (env && std::strcmp(env, "256") == 0) return 256;
  if (L != 16 || !a.bf16 || a.d_v % 32 != 0 || (a.mode == kTrainer && a.chunk < 64)) return 256;
  if (env && std::strcmp(env, "512") == 0) return 512;
  const int64_t rows = (int64_t)a.num_seqs * a.num_v_heads * a.d_v;
  const int64_t simds = device_simds();
  return rows / 4 > simds && rows / 4 <= 2 * simds ? 512 : 256;
}

// Tokens per LDS stage of the scan: 64 in a 512-thread workgroup, and for a lone wave per
// SIMD at 16 lanes per row with bf16 inputs (its 145 KiB of LDS at d_k = 128 then fits the
// one workgroup per CU it needs; measured 3.7 % faster than 32 on the long-context
// prefill), for the trainer case only when C >= 64. Chunk boundaries inside a 64-token
// stage would have to be kept in registers, and binary32 inputs double the staging
// registers: either takes the kernel past 256 registers, which ran 3.3 times slower. 32
// for 8 or 16 lanes otherwise (two workgroups per CU), 16 for 4 lanes per row.
int scan_stage_tokens(const ScanArgs &a, int L) {
  if (scan_threads(a, L) == 512) return 64;
  if (L == 16 && a.bf16 && (a.mode == kPrefill || a.chunk >= 64)) {
    const int64_t rows = (int64_t)a.num_seqs * a.num_v_heads * a.d_v;
    return rows / 4 <= device_simds() ? 64 : 32;
  }
  return L >= 8 ? 32 : 16;
}

// Rows per group of L lanes at 4 lanes per row in 256-thread workgroups: two rows (128
// per workgroup) share each token's k and q read from LDS, which halves the LDS reads per
// row; the kernel then holds up to 256 registers and 64 KiB of LDS, so two waves per SIMD
// run where one row per group runs three. Taken where there are rows for two such waves
// on every SIMD and the 128-row blocks pad d_v no more than 64-row blocks would (engine
// prefill workload: 13.9 against 14.4 ms). GDN_CPR_ROWS_PER_GROUP=1 or 2 overrides
// wherever two are admitted (the same bits either way).
int scan_rows_per_group(const ScanArgs &a, int L, int threads) {
  if (L != 4 || threads != 256) return 1;
  const char *env = std::getenv("GDN_CPR_ROWS_PER_GROUP");
  if (env && std::strcmp(env, "1") == 0) return 1;
  if (env && std::strcmp(env, "2") == 0) return 2;
  const int64_t rows = (int64_t)a.num_seqs * a.num_v_heads * a.d_v;
  const bool same_padding = (a.d_v + 127) / 128 * 2 == (a.d_v + 63) / 64;
  return same_padding && rows / 32 >= 2 * device_simds() ? 2 : 1;
}

// The backward's state pass is one dependent chain per row (no readout beside it to
// overlap), so it takes the widest rows that keep at most 2 waves per SIMD.
int bwd_state_lanes(const ScanArgs &a) {
  if (const int o = lanes_override()) return o;
  const int64_t rows = (int64_t)a.num_seqs * a.num_v_heads * a.d_v;
  const int64_t simds = device_simds();
  if (rows / 4 <= 2 * simds) return 16;
  if (rows / 8 <= 2 * simds) return 8;
  return 4;
}

// The backward sweeps each sequence's chunks in one workgroup per (sequence, value head,
// row block) when those workgroups alone occupy every compute unit (one chunk-pass
// workgroup fits per CU); otherwise it runs chunks in parallel after a state pass.
// GDN_CPR_BWD_SCHEDULE=sequences|chunks overrides; both give the same bits.
bool bwd_sequences(const gdn_shape_t *sh) {
  const char *env = std::getenv("GDN_CPR_BWD_SCHEDULE");
  if (env && std::strcmp(env, "sequences") == 0) return true;
  if (env && std::strcmp(env, "chunks") == 0) return false;
  const int64_t items = (int64_t)sh->num_seqs * sh->num_v_heads * backward_row_blocks(sh->d_v);
  return items >= device_simds() / 4;
}

// Decode streams every row once per step. For d_k >= 32 a row sits on 32 lanes, each lane
// moving 16 bytes of the row at d_k = 128 (an in-place read-modify-write stream over HBM
// measured 6.03 TB/s with 16 bytes per lane against 5.73 with 32); 16 lanes per row below.
// GDN_CPR_LANES_PER_ROW (16, 8, 4, or 32 for decode) overrides.
int decode_lanes(int d_k) {
  const char *env = std::getenv("GDN_CPR_LANES_PER_ROW");
  if (env && std::strcmp(env, "32") == 0 && d_k >= 32) return 32;
  if (const int o = lanes_override()) return o;
  return d_k >= 32 ? 32 : 16;
}

// SHA-256 of the contract text for an admitted (chunk, d_k), computed once per process and
// entry: the text is fixed for the library, and hashing it on every call would cost each
// decode step microseconds of host time.
const uint8_t *contract_digest(bool two_level, int32_t chunk, int32_t d_k) {
  static std::once_flag once[2][5][4];
  static uint8_t digest[2][5][4][32];
  const int c = __builtin_ctz((unsigned)chunk) - 4, d = __builtin_ctz((unsigned)d_k) - 4;
  std::call_once(once[two_level][c][d], [&] {
    const std::string text = two_level ? cpr2_contract_text(chunk, d_k) : contract_text(chunk, d_k);
    sha256(reinterpret_cast<const uint8_t *>(text.data()), text.size(), digest[two_level][c][d]);
  });
  return digest[two_level][c][d];
}

gdn_status_t check_shape(const char *fn, const gdn_shape_t *sh, const uint8_t *identity,
                         bool two_level = false) {
  if (!sh) return fail(GDN_E_NULL, std::string(fn) + ": shape is NULL");
  if (!identity) return fail(GDN_E_NULL, std::string(fn) + ": expected_identity is NULL");
  if (sh->num_seqs < 0 || sh->num_qk_heads < 1 || sh->num_v_heads < 1)
    return fail(GDN_E_SHAPE, std::string(fn) + ": need num_seqs >= 0 and head counts >= 1");
  if (sh->num_v_heads % sh->num_qk_heads != 0)
    return fail(GDN_E_SHAPE, std::string(fn) + ": num_v_heads must be a multiple of num_qk_heads");
  if (!admitted_dk(sh->d_k))
    return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": d_k must be 16, 32, 64 or 128");
  if (two_level && !cpr2_dk_admitted(sh->d_k))
    return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": the two-level reading admits d_k 32, 64 or 128");
  if (sh->d_v < 1 || sh->d_v > 1024)
    return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": d_v must be in [1, 1024]");
  if ((int64_t)sh->num_v_heads * (sh->d_k > sh->d_v ? sh->d_k : sh->d_v) > kMaxHeadWidth)
    return fail(GDN_E_SHAPE, std::string(fn) + ": num_v_heads * max(d_k, d_v) must be <= 2^20");
  if (!admitted_chunk(sh->chunk))
    return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": chunk must be 16, 32, 64, 128 or 256");
  if (sh->qkv_dtype != GDN_DTYPE_F32 && sh->qkv_dtype != GDN_DTYPE_BF16)
    return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": qkv_dtype must be F32 or BF16");
  if (std::memcmp(contract_digest(two_level, sh->chunk, sh->d_k), identity, 32) != 0)
    return fail(GDN_E_IDENTITY, std::string(fn) + ": expected_identity differs from this "
                                "library's contract for (chunk, d_k)");
  return GDN_OK;
}

gdn_status_t check_inputs(const char *fn, const gdn_shape_t *sh, const void *q, const void *k,
                          const void *v, const float *a, const float *b) {
  if (!q || !k || !v || !a || !b)
    return fail(GDN_E_NULL, std::string(fn) + ": q, k, v, a and b are required");
  const size_t vec = sh->qkv_dtype == GDN_DTYPE_BF16 ? 8 : 16;
  if (!aligned(q, vec) || !aligned(k, vec) || !aligned(v, sh->qkv_dtype == GDN_DTYPE_BF16 ? 2 : 4) ||
      !aligned(a, 4) || !aligned(b, 4))
    return fail(GDN_E_SHAPE, std::string(fn) + ": q and k must be " + std::to_string(vec) +
                                 "-byte aligned, v, a and b element aligned");
  return GDN_OK;
}

gdn_status_t check_state(const char *fn, const char *name, const float *p) {
  if (p && !aligned(p, 16))
    return fail(GDN_E_SHAPE, std::string(fn) + ": " + name + " must be 16-byte aligned");
  return GDN_OK;
}

gdn_status_t scan_common(const char *fn, const gdn_shape_t *sh, const uint8_t *identity,
                         const int32_t *cu, int64_t T, const void *q, const void *k,
                         const void *v, const float *a, const float *b, const float *s0,
                         float *o, ScanArgs &args, bool two_level = false) {
  gdn_status_t st = check_shape(fn, sh, identity, two_level);
  if (st != GDN_OK) return st;
  if (T < 0 || T > kMaxInt32)
    return fail(GDN_E_SHAPE, std::string(fn) + ": total_tokens must be in [0, 2^31)");
  if (sh->num_seqs > 0 && !cu) return fail(GDN_E_NULL, std::string(fn) + ": cu_seqlens is NULL");
  if (cu && !aligned(cu, 4)) return fail(GDN_E_SHAPE, std::string(fn) + ": cu_seqlens misaligned");
  if (T > 0) {
    st = check_inputs(fn, sh, q, k, v, a, b);
    if (st != GDN_OK) return st;
    if (!o) return fail(GDN_E_NULL, std::string(fn) + ": o is required");
    if (!aligned(o, 4)) return fail(GDN_E_SHAPE, std::string(fn) + ": o misaligned");
  }
  if ((st = check_state(fn, "initial_state", s0)) != GDN_OK) return st;
  args = ScanArgs{};
  args.num_seqs = sh->num_seqs;
  args.num_qk_heads = sh->num_qk_heads;
  args.num_v_heads = sh->num_v_heads;
  args.d_k = sh->d_k;
  args.d_v = sh->d_v;
  args.chunk = sh->chunk;
  args.bf16 = sh->qkv_dtype == GDN_DTYPE_BF16;
  args.total_tokens = T;
  args.cu_seqlens = cu;
  args.q = q;
  args.k = k;
  args.v = v;
  args.a = a;
  args.b = b;
  args.initial_state = s0;
  args.o = o;
  return GDN_OK;
}

gdn_status_t run_scan(const char *fn, ScanArgs &args, void *stream) {
  const int L = scan_lanes(args), threads = scan_threads(args, L);
  const int R = scan_rows_per_group(args, L, threads);
  if (scan_grid(args, L, threads, R) > kMaxInt32)
    return fail(GDN_E_SHAPE, std::string(fn) + ": num_seqs * num_v_heads * row blocks too large");
  const hipError_t e = launch_scan(args, L, scan_stage_tokens(args, L), threads, R,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return ok();
}

}  // namespace

gdn_status_t fail(gdn_status_t status, const std::string &message) {
  g_last_error = message;
  return status;
}

gdn_status_t ok() {
  g_last_error.clear();
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

GDN_EXPORT const char *gdn_last_error(void) { return gdn::g_last_error.c_str(); }

GDN_EXPORT gdn_status_t gdn_cpr_trainer_fwd(const gdn_shape_t *shape,
                                            const uint8_t *expected_identity,
                                            const int32_t *cu_seqlens, int64_t total_tokens,
                                            const void *q, const void *k, const void *v,
                                            const float *a, const float *b,
                                            const float *initial_state, float *o,
                                            float *chunk_states, int64_t total_chunks,
                                            void *stream) {
  const char *fn = "gdn_cpr_trainer_fwd";
  gdn::ScanArgs args;
  gdn_status_t st = gdn::scan_common(fn, shape, expected_identity, cu_seqlens, total_tokens, q,
                                     k, v, a, b, initial_state, o, args);
  if (st != GDN_OK) return st;
  if (total_chunks < 0 || total_chunks > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_chunks must be in [0, 2^31)");
  if (total_chunks > total_tokens / shape->chunk)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_chunks exceeds total_tokens / chunk");
  if (total_chunks > 0 && !chunk_states)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": chunk_states is required");
  if ((st = gdn::check_state(fn, "chunk_states", chunk_states)) != GDN_OK) return st;
  args.mode = gdn::kTrainer;
  args.total_chunks = total_chunks;
  args.chunk_states = chunk_states;
  return gdn::run_scan(fn, args, stream);
}

GDN_EXPORT gdn_status_t gdn_cpr_prefill(const gdn_shape_t *shape,
                                        const uint8_t *expected_identity,
                                        const int32_t *cu_seqlens, int64_t total_tokens,
                                        const void *q, const void *k, const void *v,
                                        const float *a, const float *b,
                                        const float *initial_state, float *o,
                                        float *final_state, void *stream) {
  const char *fn = "gdn_cpr_prefill";
  gdn::ScanArgs args;
  gdn_status_t st = gdn::scan_common(fn, shape, expected_identity, cu_seqlens, total_tokens, q,
                                     k, v, a, b, initial_state, o, args);
  if (st != GDN_OK) return st;
  if (shape->num_seqs > 0 && !final_state)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": final_state is required");
  if ((st = gdn::check_state(fn, "final_state", final_state)) != GDN_OK) return st;
  args.mode = gdn::kPrefill;
  args.final_state = final_state;
  return gdn::run_scan(fn, args, stream);
}

GDN_EXPORT gdn_status_t gdn_cpr_decode_step(const gdn_shape_t *shape,
                                            const uint8_t *expected_identity,
                                            const int32_t *pos, const void *q, const void *k,
                                            const void *v, const float *a, const float *b,
                                            float *state, float *o, float *resync_states,
                                            void *stream) {
  const char *fn = "gdn_cpr_decode_step";
  gdn_status_t st = gdn::check_shape(fn, shape, expected_identity);
  if (st != GDN_OK) return st;
  if (shape->num_seqs > 0) {
    if (!pos) return gdn::fail(GDN_E_NULL, std::string(fn) + ": pos is NULL");
    if ((st = gdn::check_inputs(fn, shape, q, k, v, a, b)) != GDN_OK) return st;
    if (!state || !o) return gdn::fail(GDN_E_NULL, std::string(fn) + ": state and o are required");
    if (!gdn::aligned(pos, 4) || !gdn::aligned(o, 4))
      return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": pos or o misaligned");
  }
  if ((st = gdn::check_state(fn, "state", state)) != GDN_OK) return st;
  if ((st = gdn::check_state(fn, "resync_states", resync_states)) != GDN_OK) return st;
  gdn::DecodeArgs args{};
  args.num_seqs = shape->num_seqs;
  args.num_qk_heads = shape->num_qk_heads;
  args.num_v_heads = shape->num_v_heads;
  args.d_k = shape->d_k;
  args.d_v = shape->d_v;
  args.chunk = shape->chunk;
  args.bf16 = shape->qkv_dtype == GDN_DTYPE_BF16;
  args.pos = pos;
  args.q = q;
  args.k = k;
  args.v = v;
  args.a = a;
  args.b = b;
  args.state = state;
  args.o = o;
  args.resync_states = resync_states;
  const int L = gdn::decode_lanes(shape->d_k);
  if (gdn::decode_grid(args, L) > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": num_seqs * num_v_heads * row blocks too large");
  const hipError_t e = gdn::launch_decode(args, L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return gdn::ok();
}

static gdn_status_t bwd_claims(const char *fn, const gdn_shape_t *shape, int64_t total_tokens,
                               int64_t total_chunks) {
  if (!shape) return gdn::fail(GDN_E_NULL, std::string(fn) + ": shape is NULL");
  if (!gdn::admitted_chunk(shape->chunk))
    return gdn::fail(GDN_E_UNSUPPORTED, std::string(fn) + ": chunk must be 16, 32, 64, 128 or 256");
  if (total_tokens < 0 || total_tokens > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_tokens must be in [0, 2^31)");
  if (total_chunks < 0 || total_chunks > total_tokens / (shape->chunk > 0 ? shape->chunk : 1))
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_chunks must be in [0, total_tokens / chunk]");
  return GDN_OK;
}

GDN_EXPORT gdn_status_t gdn_cpr_trainer_bwd_workspace(const gdn_shape_t *shape,
                                                      int64_t total_tokens, int64_t total_chunks,
                                                      size_t *bytes) {
  const char *fn = "gdn_cpr_trainer_bwd_workspace";
  if (!bytes) return gdn::fail(GDN_E_NULL, std::string(fn) + ": bytes is NULL");
  gdn_status_t st = bwd_claims(fn, shape, total_tokens, total_chunks);
  if (st != GDN_OK) return st;
  if (shape->num_seqs < 0 || shape->num_v_heads < 1 || !gdn::admitted_dk(shape->d_k) ||
      shape->d_v < 1 || shape->d_v > 1024)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": bad num_seqs, num_v_heads, d_k or d_v");
  *bytes = (size_t)gdn::backward_workspace(shape->num_seqs, shape->num_v_heads, shape->d_k,
                                           shape->d_v, total_tokens, total_chunks).total;
  return gdn::ok();
}

// The backward behind gdn_cpr_trainer_bwd and gdn_cpr_trainer_bwd_noalloc. workspace ==
// nullptr (with workspace_bytes == 0) selects the library's fixed scratch array, after the
// other claims and a size check.
static gdn_status_t trainer_bwd_impl(
    const char *fn, const gdn_shape_t *shape, const uint8_t *expected_identity,
    const int32_t *cu_seqlens, int64_t total_tokens, const void *q, const void *k,
    const void *v, const float *a, const float *b, const float *initial_state,
    const float *chunk_states, int64_t total_chunks, const float *d_o,
    const float *d_final_state, float *dq, float *dk, float *dv, float *da, float *db,
    float *d_initial_state, void *workspace, size_t workspace_bytes, bool fixed_scratch,
    void *stream) {
  gdn::ScanArgs fwd;  // the forward claims apply unchanged (o is dq here: any non-null f32)
  gdn_status_t st = gdn::scan_common(fn, shape, expected_identity, cu_seqlens, total_tokens, q,
                                     k, v, a, b, initial_state, dq, fwd);
  if (st != GDN_OK) return st;
  if ((st = bwd_claims(fn, shape, total_tokens, total_chunks)) != GDN_OK) return st;
  if (total_chunks > 0 && !chunk_states)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": chunk_states is required");
  if (total_tokens > 0 && (!d_o || !dq || !dk || !dv || !da || !db))
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": d_o, dq, dk, dv, da and db are required");
  if (shape->num_seqs > 0 && !d_initial_state)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": d_initial_state is required");
  const float *f32[] = {chunk_states, d_final_state, d_initial_state};
  for (const float *ptr : f32)
    if ((st = gdn::check_state(fn, "a state buffer", ptr)) != GDN_OK) return st;
  const float *f4[] = {d_o, dq, dk, dv, da, db};
  for (const float *ptr : f4)
    if (ptr && !gdn::aligned(ptr, 4))
      return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": gradient buffers must be 4-byte aligned");
  const gdn::BwdWorkspace ws = gdn::backward_workspace(
      shape->num_seqs, shape->num_v_heads, shape->d_k, shape->d_v, total_tokens, total_chunks);
  if (fixed_scratch) {
    if (ws.total > (int64_t)gdn::kNoAllocScratchBytes)
      return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": these sizes need " +
                                        std::to_string(ws.total) + " bytes of scratch; the "
                                        "fixed array holds " +
                                        std::to_string(gdn::kNoAllocScratchBytes) +
                                        " (use gdn_cpr_trainer_bwd with a workspace)");
    const hipError_t e = gdn::noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": no scratch array on this device: " +
                                         hipGetErrorString(e));
    workspace_bytes = gdn::kNoAllocScratchBytes;
  }
  if (!workspace) return gdn::fail(GDN_E_NULL, std::string(fn) + ": workspace is NULL");
  if (!gdn::aligned(workspace, 256))
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace must be 256-byte aligned");
  if ((int64_t)workspace_bytes < ws.total)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace smaller than "
                                      "gdn_cpr_trainer_bwd_workspace reports");
  if (ws.slots_max > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": too many chunks");
  gdn::BwdArgs args{};
  args.num_seqs = shape->num_seqs;
  args.num_qk_heads = shape->num_qk_heads;
  args.num_v_heads = shape->num_v_heads;
  args.d_k = shape->d_k;
  args.d_v = shape->d_v;
  args.chunk = shape->chunk;
  args.bf16 = shape->qkv_dtype == GDN_DTYPE_BF16;
  args.slots_max = (int32_t)ws.slots_max;
  args.row_blocks = gdn::backward_row_blocks(shape->d_v);
  args.total_tokens = total_tokens;
  args.total_chunks = total_chunks;
  args.cu_seqlens = cu_seqlens;
  args.q = q;
  args.k = k;
  args.v = v;
  args.a = a;
  args.b = b;
  args.initial_state = initial_state;
  args.chunk_states = chunk_states;
  args.d_o = d_o;
  args.d_final_state = d_final_state;
  args.dq = dq;
  args.dk = dk;
  args.dv = dv;
  args.da = da;
  args.db = db;
  args.d_initial_state = d_initial_state;
  char *w = static_cast<char *>(workspace);
  args.plan = reinterpret_cast<int32_t *>(w + ws.plan_off);
  args.plan_cbase = reinterpret_cast<int32_t *>(w + ws.cbase_off);
  args.dsh_bnd = reinterpret_cast<float *>(w + ws.dsh_off);
  args.partials = reinterpret_cast<float *>(w + ws.partials_off);
  if (shape->num_seqs == 0) return gdn::ok();
  const int L = gdn::bwd_state_lanes(fwd);
  const bool seq = gdn::bwd_sequences(shape);
  if (gdn::backward_state_grid(args, L) > gdn::kMaxInt32 ||
      gdn::backward_chunk_grid(args, seq) > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": grid too large");
  const hipError_t e = gdn::launch_backward(args, L, seq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_cpr_trainer_bwd(
    const gdn_shape_t *shape, const uint8_t *expected_identity, const int32_t *cu_seqlens,
    int64_t total_tokens, const void *q, const void *k, const void *v, const float *a,
    const float *b, const float *initial_state, const float *chunk_states, int64_t total_chunks,
    const float *d_o, const float *d_final_state, float *dq, float *dk, float *dv, float *da,
    float *db, float *d_initial_state, void *workspace, size_t workspace_bytes, void *stream) {
  return trainer_bwd_impl("gdn_cpr_trainer_bwd", shape, expected_identity, cu_seqlens,
                          total_tokens, q, k, v, a, b, initial_state, chunk_states, total_chunks,
                          d_o, d_final_state, dq, dk, dv, da, db, d_initial_state, workspace,
                          workspace_bytes, false, stream);
}

GDN_EXPORT gdn_status_t gdn_cpr_trainer_bwd_noalloc(
    const gdn_shape_t *shape, const uint8_t *expected_identity, const int32_t *cu_seqlens,
    int64_t total_tokens, const void *q, const void *k, const void *v, const float *a,
    const float *b, const float *initial_state, const float *chunk_states, int64_t total_chunks,
    const float *d_o, const float *d_final_state, float *dq, float *dk, float *dv, float *da,
    float *db, float *d_initial_state, void *stream) {
  return trainer_bwd_impl("gdn_cpr_trainer_bwd_noalloc", shape, expected_identity, cu_seqlens,
                          total_tokens, q, k, v, a, b, initial_state, chunk_states, total_chunks,
                          d_o, d_final_state, dq, dk, dv, da, db, d_initial_state, nullptr, 0,
                          true, stream);
}

// ------------------------------------------------------------------- two-level reading

static gdn_status_t cpr2_claims(const char *fn, const gdn_shape_t *sh, int64_t T,
                                int64_t total_chunks) {
  if (!sh) return gdn::fail(GDN_E_NULL, std::string(fn) + ": shape is NULL");
  if (T < 0 || T > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_tokens must be in [0, 2^31)");
  if (sh->chunk < 1 || total_chunks < 0 || total_chunks > T / sh->chunk)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": total_chunks must be in [0, total_tokens / chunk]");
  return GDN_OK;
}

GDN_EXPORT gdn_status_t gdn_cpr2_workspace(const gdn_shape_t *shape, int64_t total_tokens,
                                           int64_t total_chunks, int32_t decode, size_t *bytes) {
  const char *fn = "gdn_cpr2_workspace";
  if (!bytes) return gdn::fail(GDN_E_NULL, std::string(fn) + ": bytes is NULL");
  gdn_status_t st = cpr2_claims(fn, shape, decode ? 0 : total_tokens, decode ? 0 : total_chunks);
  if (st != GDN_OK) return st;
  if (shape->num_seqs < 0 || shape->num_v_heads < 1 || !gdn::cpr2_dk_admitted(shape->d_k) ||
      shape->d_v < 1 || shape->d_v > 1024)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": bad num_seqs, num_v_heads, d_k or d_v");
  *bytes = (size_t)gdn::cpr2_layout(shape->num_seqs, shape->num_v_heads, shape->d_k, shape->d_v,
                                    decode ? 0 : total_chunks, decode != 0, !decode).total;
  return gdn::ok();
}

static gdn_status_t cpr2_scan(const char *fn, bool prefill, const gdn_shape_t *shape,
                              const uint8_t *expected_identity, const int32_t *cu_seqlens,
                              int64_t total_tokens, const void *q, const void *k, const void *v,
                              const float *a, const float *b, const float *initial_state, float *o,
                              float *chunk_states, float *final_state, int64_t total_chunks,
                              void *workspace, size_t workspace_bytes, void *stream) {
  gdn::ScanArgs fwd;
  gdn_status_t st = gdn::scan_common(fn, shape, expected_identity, cu_seqlens, total_tokens, q,
                                     k, v, a, b, initial_state, o, fwd, true);
  if (st != GDN_OK) return st;
  if ((st = cpr2_claims(fn, shape, total_tokens, total_chunks)) != GDN_OK) return st;
  if ((st = gdn::check_state(fn, "chunk_states", chunk_states)) != GDN_OK) return st;
  if ((st = gdn::check_state(fn, "final_state", final_state)) != GDN_OK) return st;
  const bool trainer = !prefill;
  if (prefill && shape->num_seqs > 0 && !final_state)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": final_state is required");
  if (final_state && final_state == initial_state)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": final_state must not alias initial_state");
  if (trainer && total_chunks > 0 && !chunk_states)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": chunk_states is required");
  const gdn::Cpr2Layout ws = gdn::cpr2_layout(shape->num_seqs, shape->num_v_heads, shape->d_k,
                                              shape->d_v, total_chunks, false, !trainer);
  if (!workspace) return gdn::fail(GDN_E_NULL, std::string(fn) + ": workspace is NULL");
  if (!gdn::aligned(workspace, 256))
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace must be 256-byte aligned");
  if ((int64_t)workspace_bytes < ws.total)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace smaller than gdn_cpr2_workspace reports");
  if (total_chunks + shape->num_seqs > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": too many chunks");
  gdn::Cpr2Args args{};
  args.num_seqs = shape->num_seqs;
  args.num_qk_heads = shape->num_qk_heads;
  args.num_v_heads = shape->num_v_heads;
  args.d_k = shape->d_k;
  args.d_v = shape->d_v;
  args.chunk = shape->chunk;
  args.bf16 = shape->qkv_dtype == GDN_DTYPE_BF16;
  args.slots_max = (int32_t)(total_chunks + shape->num_seqs);
  args.total_tokens = total_tokens;
  args.total_chunks = total_chunks;
  args.cu_seqlens = cu_seqlens;
  args.q = q;
  args.k = k;
  args.v = v;
  args.a = a;
  args.b = b;
  args.initial_state = initial_state;
  args.o = o;
  char *w = static_cast<char *>(workspace);
  args.plan = reinterpret_cast<int32_t *>(w + ws.plan_off);
  args.plan_cbase = reinterpret_cast<int32_t *>(w + ws.cbase_off);
  args.trans_a = reinterpret_cast<float *>(w + ws.ta_off);
  args.trans_b = reinterpret_cast<float *>(w + ws.tb_off);
  args.chunk_states = trainer ? chunk_states : reinterpret_cast<float *>(w + ws.cs_off);
  args.final_state = final_state;
  if (shape->num_seqs == 0) return gdn::ok();
  if (gdn::cpr2_max_grid(args) > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": grid too large");
  const hipError_t e = gdn::launch_cpr2_scan(args, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_cpr2_trainer_fwd(
    const gdn_shape_t *shape, const uint8_t *expected_identity, const int32_t *cu_seqlens,
    int64_t total_tokens, const void *q, const void *k, const void *v, const float *a,
    const float *b, const float *initial_state, float *o, float *chunk_states,
    int64_t total_chunks, void *workspace, size_t workspace_bytes, void *stream) {
  return cpr2_scan("gdn_cpr2_trainer_fwd", false, shape, expected_identity, cu_seqlens,
                   total_tokens, q, k, v, a, b, initial_state, o, chunk_states, nullptr,
                   total_chunks, workspace, workspace_bytes, stream);
}

GDN_EXPORT gdn_status_t gdn_cpr2_prefill(
    const gdn_shape_t *shape, const uint8_t *expected_identity, const int32_t *cu_seqlens,
    int64_t total_tokens, const void *q, const void *k, const void *v, const float *a,
    const float *b, const float *initial_state, float *o, float *final_state,
    int64_t total_chunks, void *workspace, size_t workspace_bytes, void *stream) {
  return cpr2_scan("gdn_cpr2_prefill", true, shape, expected_identity, cu_seqlens,
                   total_tokens, q, k, v, a, b, initial_state, o, nullptr, final_state,
                   total_chunks, workspace, workspace_bytes, stream);
}

GDN_EXPORT gdn_status_t gdn_cpr2_decode_step(
    const gdn_shape_t *shape, const uint8_t *expected_identity, const int32_t *pos, const void *q,
    const void *k, const void *v, const float *a, const float *b, float *state, float *boundary,
    void *cache_k, void *cache_v, float *cache_a, float *cache_b, float *o, float *resync_states,
    void *workspace, size_t workspace_bytes, void *stream) {
  const char *fn = "gdn_cpr2_decode_step";
  gdn_status_t st = gdn::check_shape(fn, shape, expected_identity, true);
  if (st != GDN_OK) return st;
  if (shape->num_seqs > 0) {
    if (!pos) return gdn::fail(GDN_E_NULL, std::string(fn) + ": pos is NULL");
    if ((st = gdn::check_inputs(fn, shape, q, k, v, a, b)) != GDN_OK) return st;
    if (!state || !boundary || !o || !cache_k || !cache_v || !cache_a || !cache_b)
      return gdn::fail(GDN_E_NULL, std::string(fn) + ": state, boundary, o and the caches are required");
    if (!gdn::aligned(pos, 4) || !gdn::aligned(o, 4) || !gdn::aligned(cache_a, 4) ||
        !gdn::aligned(cache_b, 4) || !gdn::aligned(cache_k, 16) || !gdn::aligned(cache_v, 4))
      return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": pos, o or a cache misaligned");
  }
  const float *f16[] = {state, boundary, resync_states};
  for (const float *ptr : f16)
    if ((st = gdn::check_state(fn, "a state buffer", ptr)) != GDN_OK) return st;
  const gdn::Cpr2Layout ws = gdn::cpr2_layout(shape->num_seqs, shape->num_v_heads, shape->d_k,
                                              shape->d_v, 0, true, false);
  if (!workspace) return gdn::fail(GDN_E_NULL, std::string(fn) + ": workspace is NULL");
  if (!gdn::aligned(workspace, 256))
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace must be 256-byte aligned");
  if ((int64_t)workspace_bytes < ws.total)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": workspace smaller than gdn_cpr2_workspace reports");
  if (shape->num_seqs == 0) return gdn::ok();
  // the running rows: one token through the decode kernel (no resync of its own)
  gdn::DecodeArgs d{};
  d.num_seqs = shape->num_seqs;
  d.num_qk_heads = shape->num_qk_heads;
  d.num_v_heads = shape->num_v_heads;
  d.d_k = shape->d_k;
  d.d_v = shape->d_v;
  d.chunk = shape->chunk;
  d.bf16 = shape->qkv_dtype == GDN_DTYPE_BF16;
  d.pos = pos;
  d.q = q;
  d.k = k;
  d.v = v;
  d.a = a;
  d.b = b;
  d.state = state;
  d.o = o;
  d.resync_states = nullptr;
  const int L = gdn::decode_lanes(shape->d_k);
  gdn::Cpr2Args args{};
  args.num_seqs = shape->num_seqs;
  args.num_qk_heads = shape->num_qk_heads;
  args.num_v_heads = shape->num_v_heads;
  args.d_k = shape->d_k;
  args.d_v = shape->d_v;
  args.chunk = shape->chunk;
  args.bf16 = d.bf16;
  args.decode = 1;
  args.pos = pos;
  args.state = state;
  args.boundary = boundary;
  args.resync = resync_states;
  args.cache_k = cache_k;
  args.cache_v = cache_v;
  args.cache_a = cache_a;
  args.cache_b = cache_b;
  char *w = static_cast<char *>(workspace);
  args.plan = reinterpret_cast<int32_t *>(w + ws.plan_off);
  args.trans_a = reinterpret_cast<float *>(w + ws.ta_off);
  args.trans_b = reinterpret_cast<float *>(w + ws.tb_off);
  if (gdn::decode_grid(d, L) > gdn::kMaxInt32 || gdn::cpr2_max_grid(args) > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": grid too large");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_decode(d, L, s);
  if (e == hipSuccess) e = gdn::launch_cpr2_decode_tail(args, k, v, a, b, s);
  if (e != hipSuccess)
    return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_linear_fwd(const gdn_linear_shape_t *shape,
                                       const uint8_t *expected_identity, const void *x,
                                       const void *w, float *y, void *stream) {
  const char *fn = "gdn_linear_fwd";
  if (!shape) return gdn::fail(GDN_E_NULL, std::string(fn) + ": shape is NULL");
  if (!expected_identity)
    return gdn::fail(GDN_E_NULL, std::string(fn) + ": expected_identity is NULL");
  // the linear rule is part of every contract text, one- or two-level: accept the identity
  // of any admitted one (the digests are computed once per process)
  static const std::vector<std::array<uint8_t, GDN_CPR_IDENTITY_BYTES>> digests = [] {
    std::vector<std::array<uint8_t, GDN_CPR_IDENTITY_BYTES>> all;
    const int32_t chunks[] = {16, 32, 64, 128, 256}, dks[] = {16, 32, 64, 128};
    for (int32_t c : chunks)
      for (int32_t d : dks)
        for (int two = 0; two < 2; ++two) {
          if (two && !gdn::cpr2_dk_admitted(d)) continue;
          const std::string text = two ? gdn::cpr2_contract_text(c, d) : gdn::contract_text(c, d);
          std::array<uint8_t, GDN_CPR_IDENTITY_BYTES> digest;
          gdn::sha256(reinterpret_cast<const uint8_t *>(text.data()), text.size(), digest.data());
          all.push_back(digest);
        }
    return all;
  }();
  bool known = false;
  for (const auto &digest : digests)
    known = known || std::memcmp(digest.data(), expected_identity, digest.size()) == 0;
  if (!known)
    return gdn::fail(GDN_E_IDENTITY, std::string(fn) + ": expected_identity is not this library's "
                                         "contract");
  if (shape->m < 0 || shape->n < 0 || shape->m > gdn::kMaxInt32 || shape->n > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": m and n must be in [0, 2^31)");
  if (!gdn::linear_k_admitted(shape->k))
    return gdn::fail(GDN_E_UNSUPPORTED, std::string(fn) + ": k must be a positive multiple of 512 "
                                            "up to 2^24");
  if ((shape->x_dtype != GDN_DTYPE_F32 && shape->x_dtype != GDN_DTYPE_BF16) ||
      (shape->w_dtype != GDN_DTYPE_F32 && shape->w_dtype != GDN_DTYPE_BF16))
    return gdn::fail(GDN_E_UNSUPPORTED, std::string(fn) + ": dtypes must be F32 or BF16");
  if (shape->m == 0 || shape->n == 0) return gdn::ok();
  if (!x || !w || !y) return gdn::fail(GDN_E_NULL, std::string(fn) + ": x, w and y are required");
  if (!gdn::aligned(x, 16) || !gdn::aligned(w, 16) || !gdn::aligned(y, 4))
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": x and w must be 16-byte aligned, y 4-byte");
  gdn::LinearArgs args{};
  args.m = shape->m;
  args.n = shape->n;
  args.k = (int32_t)shape->k;
  args.x_bf16 = shape->x_dtype == GDN_DTYPE_BF16;
  args.w_bf16 = shape->w_dtype == GDN_DTYPE_BF16;
  args.x = x;
  args.w = w;
  args.y = y;
  if (gdn::linear_grid(args) > gdn::kMaxInt32)
    return gdn::fail(GDN_E_SHAPE, std::string(fn) + ": m * n too large");
  const hipError_t e = gdn::launch_linear(args, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return gdn::fail(GDN_E_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return gdn::ok();
}

}  // extern "C"
