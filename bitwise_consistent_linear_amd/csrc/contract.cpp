// Contract text and its SHA-256 identity.
//
// IsoExec identifies the numerical policy that trainer and engine run by SHA-256 digests
// and checks them at run time (IsoExec, aihirek.info, section on the contract and common
// model; agentlenshq.com, section on contract structure, "identities"). Here the digest
// covers the canonical text of the one region this library implements, for a given chunk
// size C and key width d_k; every compute entry point compares the caller's expected
// digest with it before launching anything.

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "gdn_cpr.h"
#include "internal.h"

namespace gdn {

// ----------------------------------------------------------------------------- SHA-256
// FIPS 180-4, section 6.2. The initial hash words are the first 32 bits of the fractional
// parts of the square roots of the first 8 primes and the round constants those of the
// cube roots of the first 64 primes (section 4.2.2, 5.3.3); they are computed here by
// exact integer roots rather than typed in.
namespace {

using u128 = unsigned __int128;

uint64_t first_primes(int idx) {
  int found = -1;
  for (uint64_t c = 2;; ++c) {
    bool prime = true;
    for (uint64_t d = 2; d * d <= c; ++d)
      if (c % d == 0) { prime = false; break; }
    if (prime && ++found == idx) return c;
  }
}

// floor(p^(1/r) * 2^32) mod 2^32 for r = 2 or 3, by bisection on the integer root of
// p * 2^(32 r).
uint32_t frac_root_bits(uint64_t p, int r) {
  u128 target = (u128)p << (32 * r);
  u128 lo = 0, hi = (u128)1 << 37;  // p < 2^9: root < 2^36.5, and hi^3 fits in 128 bits
  while (hi - lo > 1) {
    u128 mid = (lo + hi) / 2;
    u128 pw = mid * mid;
    if (r == 3) pw *= mid;
    if (pw <= target) lo = mid; else hi = mid;
  }
  return (uint32_t)(uint64_t)lo;
}

struct ShaConstants {
  uint32_t h0[8];
  uint32_t k[64];
};

const ShaConstants &sha_constants() {
  static ShaConstants c;
  static std::once_flag once;
  std::call_once(once, [] {
    for (int i = 0; i < 8; ++i) c.h0[i] = frac_root_bits(first_primes(i), 2);
    for (int i = 0; i < 64; ++i) c.k[i] = frac_root_bits(first_primes(i), 3);
  });
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha256_block(uint32_t h[8], const uint8_t blk[64], const uint32_t k[64]) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)blk[4 * t] << 24 | (uint32_t)blk[4 * t + 1] << 16 |
           (uint32_t)blk[4 * t + 2] << 8 | (uint32_t)blk[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    uint32_t ch = (e & f) ^ (~e & g);
    uint32_t t1 = hh + S1 + ch + k[t] + w[t];
    uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    uint32_t t2 = S0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

}  // namespace

void sha256(const uint8_t *msg, size_t len, uint8_t out[32]) {
  const ShaConstants &c = sha_constants();
  uint32_t h[8];
  std::memcpy(h, c.h0, sizeof h);
  size_t full = len / 64;
  for (size_t i = 0; i < full; ++i) sha256_block(h, msg + 64 * i, c.k);
  uint8_t tail[128] = {0};
  size_t rem = len - 64 * full;
  std::memcpy(tail, msg + 64 * full, rem);
  tail[rem] = 0x80;
  size_t tail_len = rem + 1 + 8 <= 64 ? 64 : 128;
  uint64_t bits = (uint64_t)len * 8;
  for (int i = 0; i < 8; ++i) tail[tail_len - 1 - i] = (uint8_t)(bits >> (8 * i));
  for (size_t off = 0; off < tail_len; off += 64) sha256_block(h, tail + off, c.k);
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

// ------------------------------------------------------------------------- contract text

bool admitted_chunk(int32_t c) { return c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }
bool admitted_dk(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

std::string contract_text(int32_t chunk, int32_t d_k) {
  std::string s;
  s += "contract=isoexec-gdn-cpr\n";
  s += "version=3\n";
  s += "regions=gated_delta_rule,linear\n";
  s += "region=gated_delta_rule\n";
  s += "cases=trainer_fwd,trainer_bwd,engine_prefill,engine_decode\n";
  s += "recurrence=S_t=a_t*S_{t-1}*(I-b_t*k_t*k_t^T)+b_t*v_t*k_t^T;o_t=S_t*q_t\n";
  s += "row_update=x_e=a*s_e;u=dot(x,k);d=b*(v_i-u);s_e=fma(d,k_e,x_e);o_i=dot(s,q)\n";
  s += "dot=leaves:16;leaf:contiguous d_k/16;leaf_first:mul;leaf_rest:fma ascending;"
       "combine:pairwise natural order\n";
  s += "accumulate=binary32\n";
  s += "state=binary32\n";
  s += "inputs=q,k,v:binary32|bfloat16 widened exactly;a,b:binary32 used as given\n";
  s += "output=o:binary32\n";
  s += "rounding=nearest-even;denormals=kept;fusion=explicit fma only\n";
  s += "gqa=qk_head=v_head/(Hv/Hk)\n";
  s += "chunk_state=after in-sequence index j with (j+1)%C==0;floor(T_n/C) per sequence\n";
  s += "decode_resync=state after token pos when (pos+1)%C==0\n";
  s += "cpr=one_level;rows absorb every token in order;chunk states are those rows\n";
  s += "bwd_order=reverse tokens;sh=dL/dS_final or 0;dS0=sh after the first token\n";
  s += "bwd_row=sh_e=fma(g,q_e,sh_e);pq_e=g*s_e;dh=dot(sh,k);dv_i=b*dh;pb=dh*(v_i-u);"
       "xh_e=fma(-dv_i,k_e,sh_e);pk_e=fma(-dv_i,x_e,d*sh_e);pa=dot(xh,s_prev);sh_e=a*xh_e\n";
  s += "bwd_rows=dq,dk,da,db:pairwise over rows in natural order;unpaired passes through\n";
  s += "bwd_gqa=dq,dk:value heads of the group added in ascending order\n";
  s += "region=linear\n";
  s += "linear=y[m,n]=dot(x[m,:],w[:,n]) over K;dot as above with leaf K/16;"
       "inputs=x,w:binary32|bfloat16 widened exactly;output=binary32;rows independent\n";
  s += "chunk=" + std::to_string(chunk) + "\n";
  s += "d_k=" + std::to_string(d_k) + "\n";
  return s;
}

// The two-level reading: the same region and row update, other state path.
std::string cpr2_contract_text(int32_t chunk, int32_t d_k) {
  std::string s = contract_text(chunk, d_k);
  const std::string one = "cpr=one_level;rows absorb every token in order;chunk states are those rows\n";
  const size_t at = s.find(one);
  std::string two;
  two += "cpr=two_level\n";
  two += "two_level_transition=full chunk:S_end=S_start*A_c+B_c;A_c rows from unit rows e_j with "
         "v=+0,B_c rows from +0 rows with v,through row_update over the chunk's tokens\n";
  two += "two_level_boundary=S_0=initial;S_{c+1}[i,j]=fma chain over k ascending from B_c[i,j] "
         "of S_c[i,k]*A_c[k,j];chunk states are S_{c+1}\n";
  two += "two_level_outputs=rows restart from S_c at each chunk start;o=dot(s,q) after row_update\n";
  two += "two_level_final=S after the last chunk if T_n%C==0 else the restarted rows\n";
  two += "two_level_decode=running rows from the boundary state;C-token cache;after a chunk's "
         "last token rows=boundary=resync=S_{c+1} from the cache\n";
  s.replace(at, one.size(), two);
  return s;
}

}  // namespace gdn

extern "C" {

GDN_EXPORT int32_t gdn_abi_version(void) { return GDN_CPR_ABI_VERSION; }

GDN_EXPORT gdn_status_t gdn_contract_string(int32_t chunk, int32_t d_k, char *buf,
                                            size_t buf_len, size_t *out_len) {
  if (!out_len) return gdn::fail(GDN_E_NULL, "gdn_contract_string: out_len is NULL");
  if (!gdn::admitted_chunk(chunk) || !gdn::admitted_dk(d_k))
    return gdn::fail(GDN_E_UNSUPPORTED, "gdn_contract_string: chunk or d_k not admitted");
  std::string s = gdn::contract_text(chunk, d_k);
  *out_len = s.size();
  if (buf_len < s.size() + 1) {
    if (buf && buf_len) {
      std::memcpy(buf, s.data(), buf_len);
    }
    return gdn::fail(GDN_E_SHAPE, "gdn_contract_string: buffer too small");
  }
  if (!buf) return gdn::fail(GDN_E_NULL, "gdn_contract_string: buf is NULL");
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_sha256(const void *msg, size_t len, uint8_t digest[32]) {
  if (!digest || (!msg && len > 0)) return gdn::fail(GDN_E_NULL, "gdn_sha256: NULL pointer");
  gdn::sha256(static_cast<const uint8_t *>(msg), len, digest);
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_cpr2_contract_string(int32_t chunk, int32_t d_k, char *buf,
                                                 size_t buf_len, size_t *out_len) {
  if (!out_len) return gdn::fail(GDN_E_NULL, "gdn_cpr2_contract_string: out_len is NULL");
  if (!gdn::admitted_chunk(chunk) || !gdn::cpr2_dk_admitted(d_k))
    return gdn::fail(GDN_E_UNSUPPORTED, "gdn_cpr2_contract_string: chunk or d_k not admitted");
  std::string s = gdn::cpr2_contract_text(chunk, d_k);
  *out_len = s.size();
  if (buf_len < s.size() + 1) {
    if (buf && buf_len) std::memcpy(buf, s.data(), buf_len);
    return gdn::fail(GDN_E_SHAPE, "gdn_cpr2_contract_string: buffer too small");
  }
  if (!buf) return gdn::fail(GDN_E_NULL, "gdn_cpr2_contract_string: buf is NULL");
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_cpr2_contract_identity(int32_t chunk, int32_t d_k, uint8_t digest[32]) {
  if (!digest) return gdn::fail(GDN_E_NULL, "gdn_cpr2_contract_identity: digest is NULL");
  if (!gdn::admitted_chunk(chunk) || !gdn::cpr2_dk_admitted(d_k))
    return gdn::fail(GDN_E_UNSUPPORTED, "gdn_cpr2_contract_identity: chunk or d_k not admitted");
  std::string s = gdn::cpr2_contract_text(chunk, d_k);
  gdn::sha256(reinterpret_cast<const uint8_t *>(s.data()), s.size(), digest);
  return gdn::ok();
}

GDN_EXPORT gdn_status_t gdn_contract_identity(int32_t chunk, int32_t d_k, uint8_t digest[32]) {
  if (!digest) return gdn::fail(GDN_E_NULL, "gdn_contract_identity: digest is NULL");
  if (!gdn::admitted_chunk(chunk) || !gdn::admitted_dk(d_k))
    return gdn::fail(GDN_E_UNSUPPORTED, "gdn_contract_identity: chunk or d_k not admitted");
  std::string s = gdn::contract_text(chunk, d_k);
  gdn::sha256(reinterpret_cast<const uint8_t *>(s.data()), s.size(), digest);
  return gdn::ok();
}

}  // extern "C"
