// cpr_host.cpp -- the C ABI of libcpr_gdn (declared in include/cpr_gdn.h): argument validation,
// error reporting, the numerical-policy digest and the kernel launches.  No call here synchronises
// the host or allocates device memory, except gdn_state_alloc's self-allocating mode.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/cpr_gdn.h"
#include "cpr_args.hpp"
#include "cpr_schedule.hpp"
#include "cpr_launch.hpp"

struct gdn_state {
  gdn_policy policy;
  int32_t num_slots;
  float* state;
  int64_t* pos;
  float* boundary;
  int64_t* boundary_pos;
  bool owns;
  int64_t max_wgs;   // launch-shape cap of the compute kernels (0: one workgroup per work item)
  uint32_t wait_limit;   // polls per bounded wait of the overlapped kernel (0: the default)
  void* r2_ring;         // R2 resynchronisation in decode (gdn_state_attach_r2): token ring and workspace
  void* r2_work;
  hipStream_t r2_side;   // and the second stream (default priority) and events of its step's fork and join
  hipEvent_t r2_fork;
  hipEvent_t r2_join;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return GDN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_dims(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

int validate_policy(const gdn_policy* p) {
  if (p == nullptr) return fail(GDN_EINVAL, "policy is NULL");
  if (p->h_k <= 0 || p->h_v <= 0) return fail(GDN_EINVAL, "head counts must be positive (h_k=%d h_v=%d)", p->h_k, p->h_v);
  if (p->h_v % p->h_k != 0) return fail(GDN_EINVAL, "h_v (%d) must be a multiple of h_k (%d)", p->h_v, p->h_k);
  if (p->h_v > 65535) return fail(GDN_EUNSUPPORTED, "h_v (%d) above 65535", p->h_v);
  if (p->dk <= 0 || p->dv <= 0) return fail(GDN_EINVAL, "head dims must be positive (dk=%d dv=%d)", p->dk, p->dv);
  if (p->chunk <= 0) return fail(GDN_EINVAL, "chunk must be positive (got %d)", p->chunk);
  if (p->io_dtype != GDN_F32 && p->io_dtype != GDN_BF16) return fail(GDN_EINVAL, "io_dtype %d unknown", p->io_dtype);
  if (p->state_dtype != GDN_F32 && p->state_dtype != GDN_BF16)
    return fail(GDN_EINVAL, "boundary dtype %d unknown", p->state_dtype);
  if (p->schedule != cpr::kSchedule)
    return fail(GDN_EUNSUPPORTED, "schedule %d not built (only %d)", p->schedule, cpr::kSchedule);
  if (!supported_dims(p->dk, p->dv))
    return fail(GDN_EUNSUPPORTED, "head dims dk=%d dv=%d not built (dk = dv in {16, 32, 64, 128})", p->dk, p->dv);
  return GDN_OK;
}

// ---- SHA-256, FIPS 180-4 --------------------------------------------------------------------
struct Sha256 {
  uint32_t h[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                   0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};
  uint8_t buf[64];
  size_t nbuf = 0;
  uint64_t nbits = 0;

  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

  void block(const uint8_t* p) {
    static const uint32_t K[64] = {
        0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u,
        0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u,
        0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
        0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u,
        0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
        0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
        0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
        0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = (uint32_t(p[4 * i]) << 24) | (uint32_t(p[4 * i + 1]) << 16) | (uint32_t(p[4 * i + 2]) << 8) | p[4 * i + 3];
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = hh + S1 + ch + K[i] + w[i];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + mj;
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }

  void update(const uint8_t* p, size_t n) {
    nbits += uint64_t(n) * 8;
    while (n > 0) {
      const size_t take = (64 - nbuf) < n ? (64 - nbuf) : n;
      std::memcpy(buf + nbuf, p, take);
      nbuf += take; p += take; n -= take;
      if (nbuf == 64) { block(buf); nbuf = 0; }
    }
  }

  void final(uint8_t out[32]) {
    const uint64_t bits = nbits;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (nbuf != 56) update(&zero, 1);
    uint8_t len[8];
    for (int i = 0; i < 8; ++i) len[i] = uint8_t(bits >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i) {
      out[4 * i] = uint8_t(h[i] >> 24); out[4 * i + 1] = uint8_t(h[i] >> 16);
      out[4 * i + 2] = uint8_t(h[i] >> 8); out[4 * i + 3] = uint8_t(h[i]);
    }
  }
};

void put_le32(std::string& s, int32_t v) {
  for (int i = 0; i < 4; ++i) s.push_back(char((uint32_t(v) >> (8 * i)) & 0xFF));
}

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_err.c_str(); }

// Exposed for tests of the digest primitive against a reference implementation.
int gdn_sha256(const void* data, size_t n, uint8_t out[32]) {
  if ((data == nullptr && n != 0) || out == nullptr) return fail(GDN_EINVAL, "gdn_sha256: NULL pointer");
  Sha256 s;
  s.update(static_cast<const uint8_t*>(data), n);
  s.final(out);
  return ok();
}

int gdn_policy_validate(const gdn_policy* policy) {
  const int rc = validate_policy(policy);
  return rc == GDN_OK ? ok() : rc;
}

int gdn_policy_digest(const gdn_policy* p, uint8_t out[32]) {
  if (p == nullptr || out == nullptr) return fail(GDN_EINVAL, "gdn_policy_digest: NULL pointer");
  std::string bytes = "cpr-gdn-policy-v1";
  put_le32(bytes, p->h_k);
  put_le32(bytes, p->h_v);
  put_le32(bytes, p->dk);
  put_le32(bytes, p->dv);
  put_le32(bytes, p->io_dtype);
  put_le32(bytes, p->state_dtype);
  put_le32(bytes, p->schedule);
  // chunk moves bits only when the boundary dtype rounds; otherwise it is a deployment setting
  put_le32(bytes, p->state_dtype == GDN_F32 ? 0 : p->chunk);
  put_le32(bytes, cpr::kLeaf);
  put_le32(bytes, 0);  // GQA rule: value head h reads key head h / (h_v / h_k)
  Sha256 s;
  s.update(reinterpret_cast<const uint8_t*>(bytes.data()), bytes.size());
  s.final(out);
  return ok();
}

int gdn_semantic_digest(const gdn_policy* p, uint8_t out[32]) {
  if (p == nullptr || out == nullptr) return fail(GDN_EINVAL, "gdn_semantic_digest: NULL pointer");
  std::string bytes = "cpr-gdn-semantic-v1";
  put_le32(bytes, 1);  // the gated delta rule with o_t = S_t^T q_t
  put_le32(bytes, p->h_k);
  put_le32(bytes, p->h_v);
  put_le32(bytes, p->dk);
  put_le32(bytes, p->dv);
  put_le32(bytes, 0);  // GQA rule: value head h reads key head h / (h_v / h_k)
  Sha256 s;
  s.update(reinterpret_cast<const uint8_t*>(bytes.data()), bytes.size());
  s.final(out);
  return ok();
}

int gdn_deployment_digest(const gdn_policy* p, uint8_t out[32]) {
  if (p == nullptr || out == nullptr) return fail(GDN_EINVAL, "gdn_deployment_digest: NULL pointer");
  std::string bytes = "cpr-gdn-deploy-v1";
  put_le32(bytes, p->state_dtype == GDN_F32 ? p->chunk : 0);  // with bf16 boundaries chunk is policy
  put_le32(bytes, cpr::kMappingVersion);
  Sha256 s;
  s.update(reinterpret_cast<const uint8_t*>(bytes.data()), bytes.size());
  s.final(out);
  return ok();
}

int gdn_policy_check(const uint8_t mine[32], const uint8_t theirs[32]) {
  if (mine == nullptr || theirs == nullptr) return fail(GDN_EINVAL, "gdn_policy_check: NULL digest");
  if (std::memcmp(mine, theirs, 32) != 0)
    return fail(GDN_EPOLICY, "numerical policy digests differ: refusing to run mismatched kernels");
  return ok();
}

size_t gdn_state_bytes(const gdn_policy* p, int32_t num_slots) {
  if (validate_policy(p) != GDN_OK || num_slots < 0) return 0;
  return size_t(num_slots) * size_t(p->h_v) * size_t(p->dv) * size_t(p->dk) * sizeof(float);
}

int gdn_state_alloc(const gdn_policy* policy, int32_t num_slots, float* state, int64_t* pos, size_t state_bytes,
                    float* boundary, int64_t* boundary_pos, gdn_state** out) {
  if (out == nullptr) return fail(GDN_EINVAL, "gdn_state_alloc: out is NULL");
  *out = nullptr;
  int rc = validate_policy(policy);
  if (rc != GDN_OK) return rc;
  if (num_slots <= 0) return fail(GDN_EINVAL, "num_slots must be positive (got %d)", num_slots);
  if ((boundary == nullptr) != (boundary_pos == nullptr))
    return fail(GDN_EINVAL, "boundary and boundary_pos must both be NULL or both be set");
  const size_t need = gdn_state_bytes(policy, num_slots);
  const bool self = state == nullptr && pos == nullptr;
  if (!self) {
    if (state == nullptr || pos == nullptr) return fail(GDN_EINVAL, "state and pos must both be set (or both NULL)");
    if (state_bytes != need) return fail(GDN_EINVAL, "state_bytes %zu != %zu required", state_bytes, need);
  }
  if (self) {
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&state), need);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(state)");
    e = hipMalloc(reinterpret_cast<void**>(&pos), sizeof(int64_t) * size_t(num_slots));
    if (e != hipSuccess) {
      (void)hipFree(state);
      return hip_fail(e, "hipMalloc(pos)");
    }
    e = hipMemset(state, 0, need);
    if (e == hipSuccess) e = hipMemset(pos, 0, sizeof(int64_t) * size_t(num_slots));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(state);
      (void)hipFree(pos);
      return hip_fail(e, "zero-filling the state pool");
    }
  }
  gdn_state* st = new (std::nothrow) gdn_state;
  if (st == nullptr) return fail(GDN_EINVAL, "out of host memory");
  st->policy = *policy;
  st->num_slots = num_slots;
  st->state = state;
  st->pos = pos;
  st->boundary = boundary;
  st->boundary_pos = boundary_pos;
  st->owns = self;
  st->max_wgs = 0;
  st->wait_limit = 0;
  st->r2_ring = nullptr;
  st->r2_work = nullptr;
  st->r2_side = nullptr;
  st->r2_fork = st->r2_join = nullptr;
  *out = st;
  return ok();
}

static void release_r2_streams(gdn_state* st) {
  if (st->r2_join != nullptr) (void)hipEventDestroy(st->r2_join);
  if (st->r2_fork != nullptr) (void)hipEventDestroy(st->r2_fork);
  if (st->r2_side != nullptr) (void)hipStreamDestroy(st->r2_side);
  st->r2_side = nullptr;
  st->r2_fork = st->r2_join = nullptr;
}

int gdn_state_free(gdn_state* st) {
  if (st == nullptr) return ok();
  release_r2_streams(st);
  if (st->owns) {
    (void)hipFree(st->state);
    (void)hipFree(st->pos);
  }
  delete st;
  return ok();
}

int gdn_state_set_max_workgroups(gdn_state* st, int64_t max_workgroups) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_state_set_max_workgroups: state handle is NULL");
  if (max_workgroups < 0 || max_workgroups > 0x7FFFFFFF)
    return fail(GDN_EINVAL, "gdn_state_set_max_workgroups: %lld is outside [0, 2^31)", (long long)max_workgroups);
  st->max_wgs = max_workgroups;
  return ok();
}

int gdn_state_set_wait_limit(gdn_state* st, uint32_t polls) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_state_set_wait_limit: state handle is NULL");
  st->wait_limit = polls;
  return ok();
}

int gdn_device_status(void* stream) {
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  uint32_t* word = nullptr;
  hipError_t e = cpr::wait_status_word(&word);
  if (e != hipSuccess) return hip_fail(e, "gdn_device_status: status word");
  uint32_t flags = 0;
  static const uint32_t zero = 0;
  e = hipMemcpyAsync(&flags, word, sizeof flags, hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e, "gdn_device_status: reading the status word");
  if (flags == 0) return ok();
  e = hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e, "gdn_device_status: clearing the status word");
  return fail(GDN_EHIP,
              "an overlapped prefill gave up a bounded wait (flags 0x%x:%s%s%s%s); its outputs and states are "
              "not valid",
              flags, (flags & 1u) ? " pass 1 waiting for staged inputs" : "",
              (flags & 2u) ? " pass 1 waiting for a free hand-off buffer" : "",
              (flags & 4u) ? " pass 2 waiting for a hand-off" : "",
              (flags & 8u) ? " staging waiting for a free tile buffer" : "");
}

// R2 resynchronisation needs the chunk form: bf16 io, fp32 boundaries, chunks of at most 64 tokens,
// dk = dv in {32, 64, 128}.
static int r2_policy(const gdn_policy* p, const char* who) {
  if (int rc = validate_policy(p); rc != GDN_OK) return rc;
  if (p->io_dtype != GDN_BF16 || p->state_dtype != GDN_F32 || p->chunk > 64 || p->dk != p->dv ||
      (p->dk != 32 && p->dk != 64 && p->dk != 128))
    return fail(GDN_EUNSUPPORTED, "%s: R2 needs bf16 io, fp32 boundaries, chunk <= 64 and dk = dv in {32, 64, 128}",
                who);
  return GDN_OK;
}

int64_t gdn_r2_ring_bytes(const gdn_policy* policy, int32_t num_slots) {
  if (r2_policy(policy, "gdn_r2_ring_bytes") != GDN_OK) return -1;
  if (num_slots <= 0) {
    fail(GDN_EINVAL, "gdn_r2_ring_bytes: num_slots must be positive");
    return -1;
  }
  ok();
  return cpr::r2_ring_bytes(policy->h_k, policy->h_v, policy->dk, policy->chunk, num_slots);
}

int64_t gdn_r2_workspace_bytes(const gdn_policy* policy, int32_t num_slots) {
  if (r2_policy(policy, "gdn_r2_workspace_bytes") != GDN_OK) return -1;
  if (num_slots <= 0) {
    fail(GDN_EINVAL, "gdn_r2_workspace_bytes: num_slots must be positive");
    return -1;
  }
  ok();
  return cpr::r2_workspace_bytes(policy->h_v, policy->dk, num_slots);
}

int gdn_state_attach_r2(gdn_state* st, void* ring, size_t ring_bytes, void* workspace, size_t workspace_bytes) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_state_attach_r2: state handle is NULL");
  if (ring == nullptr && workspace == nullptr) {
    st->r2_ring = st->r2_work = nullptr;
    release_r2_streams(st);
    return ok();
  }
  if (ring == nullptr || workspace == nullptr)
    return fail(GDN_EINVAL, "gdn_state_attach_r2: ring and workspace must both be set (or both NULL)");
  if (int rc = r2_policy(&st->policy, "gdn_state_attach_r2"); rc != GDN_OK) return rc;
  if (st->boundary == nullptr)
    return fail(GDN_EINVAL, "gdn_state_attach_r2: the pool needs a boundary record (the chunk-start states)");
  const int64_t rb = cpr::r2_ring_bytes(st->policy.h_k, st->policy.h_v, st->policy.dk, st->policy.chunk, st->num_slots);
  const int64_t wb = cpr::r2_workspace_bytes(st->policy.h_v, st->policy.dk, st->num_slots);
  if (int64_t(ring_bytes) < rb || int64_t(workspace_bytes) < wb)
    return fail(GDN_EINVAL, "gdn_state_attach_r2: ring %zu < %lld or workspace %zu < %lld bytes", ring_bytes,
                (long long)rb, workspace_bytes, (long long)wb);
  if ((reinterpret_cast<uintptr_t>(ring) | reinterpret_cast<uintptr_t>(workspace)) % 16 != 0)
    return fail(GDN_EINVAL, "gdn_state_attach_r2: ring and workspace must be 16-byte aligned");
  if (st->r2_side == nullptr) {
    // on the current device, which holds the pool; without one (or on failure) the decode step
    // runs in sequence on the caller's stream, and the error is cleared
    hipError_t e = hipStreamCreateWithFlags(&st->r2_side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->r2_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->r2_join, hipEventDisableTiming);
    if (e != hipSuccess) {
      release_r2_streams(st);
      (void)hipGetLastError();
    }
  }
  st->r2_ring = ring;
  st->r2_work = workspace;
  return ok();
}

float* gdn_state_data(gdn_state* st) { return st ? st->state : nullptr; }
int64_t* gdn_state_positions(gdn_state* st) { return st ? st->pos : nullptr; }

int gdn_check_cu_seqlens(const int32_t* cu, int32_t num_seqs, int64_t total_tokens) {
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0");
  if (cu == nullptr) return fail(GDN_EINVAL, "cu_seqlens is NULL");
  if (cu[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int32_t i = 0; i < num_seqs; ++i)
    if (cu[i + 1] < cu[i]) return fail(GDN_EINVAL, "cu_seqlens decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
  if (int64_t(cu[num_seqs]) != total_tokens)
    return fail(GDN_EINVAL, "cu_seqlens[%d] = %d but total_tokens = %lld", num_seqs, cu[num_seqs], (long long)total_tokens);
  return ok();
}

int64_t gdn_chunk_rows_bound(int64_t total_tokens, int32_t num_seqs, int32_t chunk) {
  if (total_tokens < 0 || num_seqs < 0 || chunk <= 0) {
    fail(GDN_EINVAL, "gdn_chunk_rows_bound: bad arguments");
    return -1;
  }
  ok();
  return total_tokens / chunk + 2 * int64_t(num_seqs);
}

int gdn_chunk_rows(const int32_t* cu, const int64_t* pos0, int32_t num_seqs, int32_t chunk, int64_t* row_offsets) {
  if (cu == nullptr || row_offsets == nullptr) return fail(GDN_EINVAL, "gdn_chunk_rows: NULL pointer");
  if (num_seqs < 0 || chunk <= 0) return fail(GDN_EINVAL, "gdn_chunk_rows: bad sizes");
  int64_t acc = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    row_offsets[i] = acc;
    const int64_t L = int64_t(cu[i + 1]) - cu[i];
    const int64_t p = pos0 ? pos0[i] : 0;
    if (L < 0 || p < 0) return fail(GDN_EINVAL, "gdn_chunk_rows: negative length or position at %d", i);
    if (L > 0) acc += 1 + (p + L - 1) / chunk - p / chunk;
  }
  row_offsets[num_seqs] = acc;
  return ok();
}

static int prefill_impl(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                        const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                        float* c_stash, float* w_stash, void* stream, void* const* events, const char* who) {
  if (st == nullptr) return fail(GDN_EINVAL, "%s: state handle is NULL", who);
  if (st->r2_ring != nullptr)
    return fail(GDN_EINVAL, "%s: the pool resynchronises under R2 (gdn_state_attach_r2); prefill it with "
                            "gdn_prefill_chunked(GDN_CHUNKED_R2)", who);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "%s: negative sizes", who);
  if (total_tokens >= (int64_t(1) << 31)) return fail(GDN_EINVAL, "%s: total_tokens must fit int32 cu_seqlens", who);
  if (num_seqs > 0 && (cu_seqlens == nullptr || slot_ids == nullptr))
    return fail(GDN_EINVAL, "%s: cu_seqlens/slot_ids NULL", who);
  if (from_state != 0 && from_state != 1) return fail(GDN_EINVAL, "%s: from_state must be 0 or 1", who);
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || a == nullptr || b == nullptr || o == nullptr))
    return fail(GDN_EINVAL, "%s: token tensor NULL", who);
  const gdn_policy& P = st->policy;
  const int64_t bound = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  if (num_seqs > 0 && chunk_states == nullptr) return fail(GDN_EINVAL, "%s: chunk_states is NULL", who);
  if (chunk_state_rows < bound)
    return fail(GDN_EINVAL, "%s: chunk_state_rows %lld < bound %lld", who, (long long)chunk_state_rows,
                (long long)bound);
  if (bound > 0x7FFFFFFF) return fail(GDN_EUNSUPPORTED, "%s: too many chunks for one launch", who);
  if (reinterpret_cast<uintptr_t>(c_stash) % 16 != 0) return fail(GDN_EINVAL, "%s: c stash must be 16-byte aligned", who);
  cpr::PrefillArgs A{};
  A.max_wgs = st->max_wgs;
  A.cu = cu_seqlens;
  A.slot_ids = slot_ids;
  A.pos = st->pos;
  A.pos_out = st->pos;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.state = st->state;
  A.chunk_states = chunk_states;
  A.total_tokens = total_tokens;
  A.rows_cap = bound < chunk_state_rows ? bound : chunk_state_rows;   // rows any plan can use
  A.num_seqs = num_seqs;
  A.num_slots = st->num_slots;
  A.from_state = from_state;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.round_boundary = P.state_dtype == GDN_BF16;
  A.c_stash = total_tokens > 0 ? c_stash : nullptr;
  A.w_stash = total_tokens > 0 ? w_stash : nullptr;
  A.events = events;
  const hipError_t e = cpr::launch_prefill(P.dk, P.dv, P.io_dtype, A, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int gdn_prefill(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                float* c_stash, void* stream, void* const* events) {
  return prefill_impl(st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v, a, b, o, chunk_states,
                      chunk_state_rows, c_stash, nullptr, stream, events, "gdn_prefill");
}

int gdn_prefill_static(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                       const float* a, const float* b, void* o, void* stream, void* const* events) {
  static const char* who = "gdn_prefill_static";
  if (st == nullptr) return fail(GDN_EINVAL, "%s: state handle is NULL", who);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "%s: negative sizes", who);
  const gdn_policy& P = st->policy;
  const int64_t rows = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  const int64_t plane = int64_t(P.h_v) * P.dv * P.dk * 4;
  const int64_t rows_bytes = (rows * plane + 255) / 256 * 256;
  const int64_t stash_bytes = total_tokens * P.h_v * int64_t(P.dv) * 4;
  const int64_t cap = int64_t(cpr::kStaticScratchBytes);
  if (rows < 0 || rows_bytes > cap)
    return fail(GDN_EINVAL,
                "%s: %lld chunk-state rows of %lld bytes need %lld bytes of scratch, above the library's static "
                "%lld; split the batch or use gdn_prefill with caller-owned chunk states",
                who, (long long)rows, (long long)plane, (long long)rows_bytes, (long long)cap);
  void* scratch = nullptr;
  const hipError_t e = cpr::static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "gdn_prefill_static: static scratch");
  // the chunk-start rows first; the c stash after them when it fits too (the same bits either way)
  float* rows_ptr = static_cast<float*>(scratch);
  float* stash = total_tokens > 0 && rows_bytes + stash_bytes <= cap
                     ? reinterpret_cast<float*>(static_cast<char*>(scratch) + rows_bytes)
                     : nullptr;
  return prefill_impl(st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v, a, b, o, rows_ptr,
                      rows, stash, nullptr, stream, events, who);
}

int gdn_trainer_forward(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                        const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                        float* cw, void* stream, void* const* events) {
  if (total_tokens > 0 && cw == nullptr) return fail(GDN_EINVAL, "gdn_trainer_forward: cw is NULL");
  // pass 1 keeps every token's c in block 0 and w in block 1; pass 2 applies the kept c
  float* w = cw == nullptr || st == nullptr ? nullptr : cw + total_tokens * st->policy.h_v * int64_t(st->policy.dv);
  return prefill_impl(st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v, a, b, o, chunk_states,
                      chunk_state_rows, cw, w, stream, events, "gdn_trainer_forward");
}

// The single-launch prefills: the one-pass kernel, or pass 1 with the chunk outputs overlapped
// (chunks up to the overlap kernel's limit; longer chunks take the one-pass kernel, same bits).
static int onepass_impl(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                        const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                        void* stream, void* const* events, bool overlap, const char* who) {
  if (st == nullptr) return fail(GDN_EINVAL, "%s: state handle is NULL", who);
  if (st->r2_ring != nullptr)
    return fail(GDN_EINVAL, "%s: the pool resynchronises under R2 (gdn_state_attach_r2); prefill it with "
                            "gdn_prefill_chunked(GDN_CHUNKED_R2)", who);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "%s: negative sizes", who);
  if (total_tokens >= (int64_t(1) << 31))
    return fail(GDN_EINVAL, "%s: total_tokens must fit int32 cu_seqlens", who);
  if (num_seqs > 0 && (cu_seqlens == nullptr || slot_ids == nullptr))
    return fail(GDN_EINVAL, "%s: cu_seqlens/slot_ids NULL", who);
  if (from_state != 0 && from_state != 1) return fail(GDN_EINVAL, "%s: from_state must be 0 or 1", who);
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || a == nullptr || b == nullptr || o == nullptr))
    return fail(GDN_EINVAL, "%s: token tensor NULL", who);
  const gdn_policy& P = st->policy;
  const int64_t bound = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  if (chunk_states != nullptr && chunk_state_rows < bound)
    return fail(GDN_EINVAL, "%s: chunk_state_rows %lld < bound %lld", who, (long long)chunk_state_rows,
                (long long)bound);
  cpr::PrefillArgs A{};
  A.max_wgs = st->max_wgs;
  A.cu = cu_seqlens;
  A.slot_ids = slot_ids;
  A.pos = st->pos;
  A.pos_out = st->pos;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.state = st->state;
  A.chunk_states = chunk_states;
  A.total_tokens = total_tokens;
  A.rows_cap = chunk_states != nullptr ? (bound < chunk_state_rows ? bound : chunk_state_rows) : 0;
  A.num_seqs = num_seqs;
  A.num_slots = st->num_slots;
  A.from_state = from_state;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.round_boundary = P.state_dtype == GDN_BF16;
  A.c_stash = nullptr;
  A.w_stash = nullptr;
  A.events = events;
  A.wait_limit = st->wait_limit;
  const bool overlapped = overlap && P.chunk <= cpr::overlap_max_chunk() && cpr::overlap_fits(P.dk, P.dv, A);
  const hipError_t e = overlapped
                           ? cpr::launch_prefill_overlap(P.dk, P.dv, P.io_dtype, A, static_cast<hipStream_t>(stream))
                           : cpr::launch_prefill_fused(P.dk, P.dv, P.io_dtype, A, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int gdn_prefill_fused(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                      const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                      void* stream, void* const* events) {
  return onepass_impl(st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v, a, b, o, chunk_states,
                      chunk_state_rows, stream, events, false, "gdn_prefill_fused");
}

int gdn_prefill_overlapped(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                           const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                           const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                           void* stream, void* const* events) {
  return onepass_impl(st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v, a, b, o, chunk_states,
                      chunk_state_rows, stream, events, true, "gdn_prefill_overlapped");
}

int gdn_decode_step(gdn_state* st, const int32_t* slot_ids, int32_t batch, const void* q, const void* k,
                    const void* v, const float* a, const float* b, void* o, void* stream,
                    void* const* events) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_decode_step: state handle is NULL");
  if (batch < 0) return fail(GDN_EINVAL, "gdn_decode_step: negative batch");
  if (batch > 0 && (slot_ids == nullptr || q == nullptr || k == nullptr || v == nullptr || a == nullptr ||
                    b == nullptr || o == nullptr))
    return fail(GDN_EINVAL, "gdn_decode_step: NULL pointer");
  const gdn_policy& P = st->policy;
  cpr::DecodeArgs A{};
  A.max_wgs = st->max_wgs;
  A.slot_ids = slot_ids;
  A.pos = st->pos;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.state = st->state;
  A.boundary = st->boundary;
  A.boundary_pos = st->boundary_pos;
  A.batch = batch;
  A.num_slots = st->num_slots;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.round_boundary = P.state_dtype == GDN_BF16;
  A.events = events;
  const hipError_t e = st->r2_ring != nullptr
                           ? cpr::launch_decode_r2(P.dk, A, st->r2_ring, st->r2_work, static_cast<hipStream_t>(stream),
                                                   st->r2_side, st->r2_fork, st->r2_join)
                           : cpr::launch_decode(P.dk, P.dv, P.io_dtype, A, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_decode_step launch");
  return ok();
}

int gdn_state_resync(gdn_state* st, const int32_t* slot_ids, int32_t n, void* stream) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_state_resync: state handle is NULL");
  if (st->r2_ring != nullptr)
    return fail(GDN_EINVAL, "gdn_state_resync: the pool resynchronises under R2 inside gdn_decode_step");
  if (n < 0) return fail(GDN_EINVAL, "gdn_state_resync: negative count");
  if (n > 0 && slot_ids == nullptr) return fail(GDN_EINVAL, "gdn_state_resync: slot_ids is NULL");
  const gdn_policy& P = st->policy;
  cpr::DecodeArgs A{};
  A.max_wgs = st->max_wgs;
  A.slot_ids = slot_ids;
  A.pos = st->pos;
  A.state = st->state;
  A.boundary = st->boundary;
  A.boundary_pos = st->boundary_pos;
  A.batch = n;
  A.num_slots = st->num_slots;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.round_boundary = P.state_dtype == GDN_BF16;
  const hipError_t e = cpr::launch_resync(P.dk, P.dv, A, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_state_resync launch");
  return ok();
}

static int64_t backward_rows(int64_t total_tokens, int32_t num_seqs, int32_t chunk) {
  return total_tokens / chunk + num_seqs;   // sum over sequences of ceil(L_i / C), bounded
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// The chunk-gradient kernel's tile is 64 tokens.  Under fp32 boundaries the gradients are always
// taken at chunk 64: a forward at any other chunk is differentiated on a 64-token stash that pass 1
// recomputes from each sequence's first row.  A chunk-start state does not depend on C there, so
// those rows are the bits a 64-token forward would have stored, and the gradients are the same bits
// whatever C the forward ran at (C is a deployment setting, as the policy digest says).  Under
// bf16 boundaries C is numerical policy and the gradients run at min(C, 64) on the forward's own
// (rounded) rows.
constexpr int32_t kGradTile = 64;

static bool rebuilds_stash(const gdn_policy& P) { return P.state_dtype == GDN_F32 && P.chunk != kGradTile; }

static int32_t grad_chunk_of(const gdn_policy& P) {
  return P.state_dtype == GDN_F32 ? kGradTile : (P.chunk < kGradTile ? P.chunk : kGradTile);
}

// Workspace beyond the gradient passes' own when the stash is rebuilt: the 64-token stash, a slot
// id per sequence and a position per row of the forward's stash.
static int64_t rechunk_bytes(const gdn_policy& P, int64_t total_tokens, int32_t num_seqs) {
  if (!rebuilds_stash(P)) return 0;
  const int64_t plane = int64_t(P.dk) * P.dv;
  return align256(backward_rows(total_tokens, num_seqs, kGradTile) * P.h_v * plane * 4) +
         align256(int64_t(num_seqs) * 4) + align256(backward_rows(total_tokens, num_seqs, P.chunk) * 8);
}

int64_t gdn_backward_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs) {
  if (gdn_policy_validate(policy) != GDN_OK) return -1;
  if (total_tokens < 0 || num_seqs < 0) {
    fail(GDN_EINVAL, "gdn_backward_workspace_bytes: negative sizes");
    return -1;
  }
  const gdn_policy& P = *policy;
  const int64_t plane = int64_t(P.dk) * P.dv;
  const int32_t chunk = grad_chunk_of(P);   // the gradient passes' chunk
  const int64_t adj_rows = backward_rows(total_tokens, num_seqs, chunk) + num_seqs;
  const int64_t adj = adj_rows * P.h_v * plane * 4;
  const int64_t per_token = total_tokens * P.h_v * int64_t(P.dv) * 4;
  const int64_t parts = adj_rows * P.h_v * cpr::adjoint_parts(P.dk) * 8;
  const int64_t xv = total_tokens * P.h_v * 4;
  ok();
  return align256(adj) + 3 * align256(per_token) + align256(parts) + align256(xv) +
         rechunk_bytes(P, total_tokens, num_seqs);
}

int gdn_backward(const gdn_policy* policy, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                 const void* q, const void* k, const void* v, const float* a, const float* b,
                 const float* chunk_states, int64_t chunk_state_rows, const float* cw, const void* d_o,
                 const float* d_state,
                 float* dq, float* dk, float* dv, float* da, float* db, float* d_state0, void* workspace,
                 size_t workspace_bytes, void* stream, void* const* events) {
  if (int rc = gdn_policy_validate(policy); rc != GDN_OK) return rc;
  const gdn_policy& P = *policy;
  if (P.chunk > kGradTile && P.state_dtype != GDN_F32)
    return fail(GDN_EUNSUPPORTED, "gdn_backward: chunk %d > %d with bf16 boundaries", P.chunk, kGradTile);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "gdn_backward: negative sizes");
  if (total_tokens >= (int64_t(1) << 31))
    return fail(GDN_EINVAL, "gdn_backward: total_tokens must fit int32 cu_seqlens");
  if (num_seqs > 0 && cu_seqlens == nullptr) return fail(GDN_EINVAL, "gdn_backward: cu_seqlens is NULL");
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || a == nullptr || b == nullptr ||
                           d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || da == nullptr ||
                           db == nullptr))
    return fail(GDN_EINVAL, "gdn_backward: token tensor NULL");
  const int64_t rows = backward_rows(total_tokens, num_seqs, P.chunk);
  if (num_seqs > 0 && chunk_states == nullptr) return fail(GDN_EINVAL, "gdn_backward: chunk_states is NULL");
  if (num_seqs > 0 && chunk_state_rows < rows)
    return fail(GDN_EINVAL, "gdn_backward: chunk_state_rows %lld < %lld", (long long)chunk_state_rows,
                (long long)rows);
  if (rows * P.h_k > 0x7FFFFFFF) return fail(GDN_EUNSUPPORTED, "gdn_backward: too many chunks for one launch");
  const int64_t need = gdn_backward_workspace_bytes(policy, total_tokens, num_seqs);
  if (need < 0) return GDN_EINVAL;
  if (int64_t(workspace_bytes) < need || (need > 0 && workspace == nullptr))
    return fail(GDN_EINVAL, "gdn_backward: workspace of %lld bytes < %lld", (long long)workspace_bytes,
                (long long)need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return fail(GDN_EINVAL, "gdn_backward: workspace must be 16-byte aligned");
  const int64_t plane = int64_t(P.dk) * P.dv;
  const int32_t chunk = grad_chunk_of(P);   // the gradient passes' chunk
  const int64_t rows_g = backward_rows(total_tokens, num_seqs, chunk);
  if (rows_g * P.h_k > 0x7FFFFFFF) return fail(GDN_EUNSUPPORTED, "gdn_backward: too many chunks for one launch");
  const int64_t adj_bytes = align256((rows_g + num_seqs) * P.h_v * plane * 4);
  const int64_t tok_bytes = align256(total_tokens * P.h_v * int64_t(P.dv) * 4);
  const int64_t part_bytes = align256((rows_g + num_seqs) * P.h_v * cpr::adjoint_parts(P.dk) * 8) +
                             align256(total_tokens * P.h_v * 4);   // and v_t . dv_t per token-head
  char* ws = static_cast<char*>(workspace);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const float* stash = chunk_states;
  if (rebuilds_stash(P) && num_seqs > 0) {
    // the 64-token stash: pass 1 from each sequence's first row of the caller's stash
    char* xs = ws + adj_bytes + 3 * tok_bytes + part_bytes;
    float* fine = reinterpret_cast<float*>(xs);
    int32_t* ids = reinterpret_cast<int32_t*>(xs + align256(rows_g * P.h_v * plane * 4));
    int64_t* pos = reinterpret_cast<int64_t*>(reinterpret_cast<char*>(ids) + align256(int64_t(num_seqs) * 4));
    cpr::BackwardArgs R{};
    R.cu = cu_seqlens;
    R.total_tokens = total_tokens;
    R.num_seqs = num_seqs;
    R.chunk = P.chunk;
    R.rows_cap = rows;
    hipError_t e = cpr::launch_rechunk_setup(R, ids, pos, hs);
    if (e != hipSuccess) return hip_fail(e, "gdn_backward re-chunk setup");
    cpr::PrefillArgs F{};
    F.cu = cu_seqlens;
    F.slot_ids = ids;
    F.pos = pos;
    F.pos_out = pos;
    F.q = q; F.k = k; F.v = v; F.a = a; F.b = b;
    F.o = nullptr;
    F.state = const_cast<float*>(chunk_states);    // read only: every sequence continues from its row 0
    F.chunk_states = fine;
    F.total_tokens = total_tokens;
    F.rows_cap = rows_g;
    F.num_seqs = num_seqs;
    F.num_slots = static_cast<int32_t>(rows);
    F.from_state = 1;
    F.h_k = P.h_k; F.h_v = P.h_v; F.chunk = kGradTile;
    F.round_boundary = 0;
    e = cpr::launch_boundary_pass(P.dk, P.dv, P.io_dtype, F, hs);
    if (e != hipSuccess) return hip_fail(e, "gdn_backward re-chunk pass");
    stash = fine;
  }
  cpr::BackwardArgs A{};
  A.cu = cu_seqlens;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b;
  A.d_o = d_o;
  A.d_state = d_state;
  A.chunk_states = stash;
  A.adjoint = reinterpret_cast<float*>(ws);
  A.dc = reinterpret_cast<float*>(ws + adj_bytes);
  A.cc = reinterpret_cast<float*>(ws + adj_bytes + tok_bytes);
  A.ww = reinterpret_cast<float*>(ws + adj_bytes + 2 * tok_bytes);
  A.hpart = reinterpret_cast<double*>(ws + adj_bytes + 3 * tok_bytes);
  A.xv = reinterpret_cast<float*>(ws + adj_bytes + 3 * tok_bytes +
                                  align256((rows_g + num_seqs) * P.h_v * cpr::adjoint_parts(P.dk) * 8));
  A.have_cw = cw != nullptr;
  A.hparts = cpr::adjoint_parts(P.dk);
  if (cw != nullptr) {                       // the trainer forward's c and w: no replay needed
    A.cc = const_cast<float*>(cw);
    A.ww = const_cast<float*>(cw) + total_tokens * P.h_v * int64_t(P.dv);
  }
  A.dq = dq; A.dk = dk; A.dv = dv; A.da = da; A.db = db;
  A.d_state0 = d_state0;
  A.total_tokens = total_tokens;
  A.rows_cap = rows_g;
  A.adj_rows = rows_g + num_seqs;
  A.num_seqs = num_seqs;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = chunk;
  A.events = events;
  const hipError_t e = cpr::launch_backward(P.dk, P.dv, P.io_dtype, A, hs);
  if (e != hipSuccess) return hip_fail(e, "gdn_backward launch");
  return ok();
}

int64_t gdn_prefill_chunked_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs) {
  if (gdn_policy_validate(policy) != GDN_OK) return -1;
  if (total_tokens < 0 || num_seqs < 0) {
    fail(GDN_EINVAL, "gdn_prefill_chunked_workspace_bytes: negative sizes");
    return -1;
  }
  const int64_t per = cpr::chunked_workspace_floats(policy->dk);
  if (per == 0 || policy->dk != policy->dv) {
    fail(GDN_EUNSUPPORTED, "gdn_prefill_chunked: head dims %d x %d not built", policy->dk, policy->dv);
    return -1;
  }
  ok();
  return gdn_chunk_rows_bound(total_tokens, num_seqs, policy->chunk) * policy->h_v * per * 4;
}

// The chunkwise evaluation behind gdn_prefill_chunked and gdn_trainer_forward_chunked; `bwd`
// (nullable) is the trainer forward's stash past the workspace: T^T and W^T per chunk row and value
// head, then every token's c.
static int chunked_call(const char* fn, gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, const int32_t* slot_ids, int32_t from_state, const void* q,
                        const void* k, const void* v, const float* a, const float* b, void* o, float* chunk_states,
                        int64_t chunk_state_rows, int32_t outputs, void* workspace, size_t workspace_bytes,
                        float* bwd, void* stream, void* const* events) {
  if (st == nullptr) return fail(GDN_EINVAL, "%s: state handle is NULL", fn);
  const gdn_policy& P = st->policy;
  if (P.io_dtype != GDN_BF16) return fail(GDN_EUNSUPPORTED, "%s: bf16 io only", fn);
  if (P.state_dtype != GDN_F32) return fail(GDN_EUNSUPPORTED, "%s: fp32 boundary dtype only", fn);
  if (P.chunk > 64) return fail(GDN_EUNSUPPORTED, "%s: chunk %d > 64", fn, P.chunk);
  if (outputs != GDN_CHUNKED_NATIVE && outputs != GDN_CHUNKED_R2)
    return fail(GDN_EINVAL, "%s: outputs must be GDN_CHUNKED_NATIVE or GDN_CHUNKED_R2", fn);
  if (outputs == GDN_CHUNKED_NATIVE && st->r2_ring != nullptr)
    return fail(GDN_EINVAL, "%s: the pool resynchronises under R2; native outputs would leave its ring behind", fn);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "%s: negative sizes", fn);
  if (total_tokens >= (int64_t(1) << 31)) return fail(GDN_EINVAL, "%s: total_tokens must fit int32 cu_seqlens", fn);
  if (num_seqs > 0 && (cu_seqlens == nullptr || slot_ids == nullptr))
    return fail(GDN_EINVAL, "%s: cu_seqlens/slot_ids NULL", fn);
  if (from_state != 0 && from_state != 1) return fail(GDN_EINVAL, "%s: from_state must be 0 or 1", fn);
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || a == nullptr || b == nullptr || o == nullptr))
    return fail(GDN_EINVAL, "%s: token tensor NULL", fn);
  const int64_t bound = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  if (num_seqs > 0 && chunk_states == nullptr) return fail(GDN_EINVAL, "%s: chunk_states is NULL", fn);
  if (chunk_state_rows < bound)
    return fail(GDN_EINVAL, "%s: chunk_state_rows %lld < bound %lld", fn, (long long)chunk_state_rows,
                (long long)bound);
  if (bound * P.h_k > 0x7FFFFFFF) return fail(GDN_EUNSUPPORTED, "%s: too many chunks for one launch", fn);
  const int64_t need = gdn_prefill_chunked_workspace_bytes(&P, total_tokens, num_seqs);
  if (need < 0) return GDN_EUNSUPPORTED;
  if (int64_t(workspace_bytes) < need || (need > 0 && workspace == nullptr))
    return fail(GDN_EINVAL, "%s: workspace of %lld bytes < %lld", fn, (long long)workspace_bytes, (long long)need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return fail(GDN_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  cpr::PrefillArgs A{};
  A.max_wgs = st->max_wgs;
  A.cu = cu_seqlens;
  A.slot_ids = slot_ids;
  A.pos = st->pos;
  A.pos_out = st->pos;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.state = st->state;
  A.chunk_states = chunk_states;
  A.total_tokens = total_tokens;
  A.rows_cap = bound;
  A.num_seqs = num_seqs;
  A.num_slots = st->num_slots;
  A.from_state = from_state;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.round_boundary = 0;
  A.c_stash = nullptr;
  A.w_stash = nullptr;
  A.events = events;
  if (bwd != nullptr) {
    A.chunk_bwd = bwd;
    A.c_stash = bwd + bound * P.h_v * cpr::chunked_bwd_floats(P.dk);
  }
  if (outputs == GDN_CHUNKED_R2 && st->r2_ring != nullptr) {
    A.r2_ring = st->r2_ring;
    A.r2_boundary = st->boundary;
    A.r2_boundary_pos = st->boundary_pos;
  }
  const hipError_t e = cpr::launch_prefill_chunked(P.dk, P.dv, 1, A, workspace, outputs,
                                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, (std::string(fn) + " launch").c_str());
  return ok();
}

int gdn_prefill_chunked(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state, const void* q, const void* k, const void* v,
                        const float* a, const float* b, void* o, float* chunk_states, int64_t chunk_state_rows,
                        int32_t outputs, void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  return chunked_call("gdn_prefill_chunked", st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q, k, v,
                      a, b, o, chunk_states, chunk_state_rows, outputs, workspace, workspace_bytes, nullptr, stream,
                      events);
}

// The chunkwise trainer forward keeps, in one stash: the chunk form's workspace, then T^T and W^T
// per chunk row and value head, then every token's c.
static int64_t chunked_stash_parts(const gdn_policy& P, int64_t total_tokens, int32_t num_seqs, int64_t* ws_bytes,
                                   int64_t* bwd_bytes) {
  const int64_t rows = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  *ws_bytes = align256(rows * P.h_v * cpr::chunked_workspace_floats(P.dk) * 4);
  *bwd_bytes = rows * P.h_v * cpr::chunked_bwd_floats(P.dk) * 4 + total_tokens * P.h_v * int64_t(P.dv) * 4;
  return *ws_bytes + align256(*bwd_bytes);
}

int64_t gdn_trainer_forward_chunked_stash_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs) {
  if (gdn_prefill_chunked_workspace_bytes(policy, total_tokens, num_seqs) < 0) return -1;
  int64_t ws, bw;
  const int64_t n = chunked_stash_parts(*policy, total_tokens, num_seqs, &ws, &bw);
  ok();
  return n;
}

int gdn_trainer_forward_chunked(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                const int32_t* slot_ids, int32_t from_state, const void* q, const void* k,
                                const void* v, const float* a, const float* b, void* o, float* chunk_states,
                                int64_t chunk_state_rows, void* stash, size_t stash_bytes, void* stream,
                                void* const* events) {
  if (st == nullptr) return fail(GDN_EINVAL, "gdn_trainer_forward_chunked: state handle is NULL");
  const int64_t need = gdn_trainer_forward_chunked_stash_bytes(&st->policy, total_tokens, num_seqs);
  if (need < 0) return GDN_EUNSUPPORTED;
  if (int64_t(stash_bytes) < need || (need > 0 && stash == nullptr))
    return fail(GDN_EINVAL, "gdn_trainer_forward_chunked: stash of %lld bytes < %lld", (long long)stash_bytes,
                (long long)need);
  int64_t ws, bw;
  chunked_stash_parts(st->policy, total_tokens, num_seqs, &ws, &bw);
  float* bwd = reinterpret_cast<float*>(static_cast<char*>(stash) + ws);
  return chunked_call("gdn_trainer_forward_chunked", st, cu_seqlens, num_seqs, total_tokens, slot_ids, from_state, q,
                      k, v, a, b, o, chunk_states, chunk_state_rows, GDN_CHUNKED_NATIVE, stash, size_t(ws), bwd,
                      stream, events);
}

int64_t gdn_backward_chunked_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs) {
  if (gdn_prefill_chunked_workspace_bytes(policy, total_tokens, num_seqs) < 0) return -1;
  const gdn_policy& P = *policy;
  const int64_t plane = int64_t(P.dk) * P.dv;
  const int64_t adj_rows = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk) + num_seqs;
  const int64_t per_token = total_tokens * P.h_v * int64_t(P.dv) * 4;
  ok();
  return align256(adj_rows * P.h_v * plane * 4) + 2 * align256(per_token) +
         align256(adj_rows * P.h_v * cpr::backward_chunked_parts(P.dk) * 8) + align256(total_tokens * P.h_v * 4);
}

int gdn_backward_chunked(const gdn_policy* policy, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         const void* q, const void* k, const void* v, const float* a, const float* b,
                         const float* chunk_states, int64_t chunk_state_rows, const void* stash, size_t stash_bytes,
                         const void* d_o, const float* d_state, float* dq, float* dk, float* dv, float* da, float* db,
                         float* d_state0, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* events) {
  const char* fn = "gdn_backward_chunked";
  if (int rc = gdn_policy_validate(policy); rc != GDN_OK) return rc;
  const gdn_policy& P = *policy;
  if (P.io_dtype != GDN_BF16) return fail(GDN_EUNSUPPORTED, "%s: bf16 io only", fn);
  if (P.state_dtype != GDN_F32) return fail(GDN_EUNSUPPORTED, "%s: fp32 boundary dtype only", fn);
  if (P.chunk > 64) return fail(GDN_EUNSUPPORTED, "%s: chunk %d > 64", fn, P.chunk);
  const int64_t need_stash = gdn_trainer_forward_chunked_stash_bytes(policy, total_tokens, num_seqs);
  const int64_t need = gdn_backward_chunked_workspace_bytes(policy, total_tokens, num_seqs);
  if (need_stash < 0 || need < 0) return GDN_EUNSUPPORTED;
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_EINVAL, "%s: negative sizes", fn);
  if (total_tokens >= (int64_t(1) << 31)) return fail(GDN_EINVAL, "%s: total_tokens must fit int32 cu_seqlens", fn);
  if (num_seqs > 0 && cu_seqlens == nullptr) return fail(GDN_EINVAL, "%s: cu_seqlens is NULL", fn);
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || a == nullptr || b == nullptr ||
                           d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || da == nullptr ||
                           db == nullptr))
    return fail(GDN_EINVAL, "%s: token tensor NULL", fn);
  const int64_t rows = gdn_chunk_rows_bound(total_tokens, num_seqs, P.chunk);
  if (num_seqs > 0 && chunk_states == nullptr) return fail(GDN_EINVAL, "%s: chunk_states is NULL", fn);
  if (num_seqs > 0 && chunk_state_rows < rows)
    return fail(GDN_EINVAL, "%s: chunk_state_rows %lld < %lld", fn, (long long)chunk_state_rows, (long long)rows);
  if (rows * P.h_k > 0x7FFFFFFF) return fail(GDN_EUNSUPPORTED, "%s: too many chunks for one launch", fn);
  if (int64_t(stash_bytes) < need_stash || (need_stash > 0 && stash == nullptr))
    return fail(GDN_EINVAL, "%s: stash of %lld bytes < %lld", fn, (long long)stash_bytes, (long long)need_stash);
  if (int64_t(workspace_bytes) < need || (need > 0 && workspace == nullptr))
    return fail(GDN_EINVAL, "%s: workspace of %lld bytes < %lld", fn, (long long)workspace_bytes, (long long)need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0 || (reinterpret_cast<uintptr_t>(stash) & 15) != 0)
    return fail(GDN_EINVAL, "%s: workspace and stash must be 16-byte aligned", fn);
  const int64_t plane = int64_t(P.dk) * P.dv;
  const int64_t adj_bytes = align256((rows + num_seqs) * P.h_v * plane * 4);
  const int64_t tok_bytes = align256(total_tokens * P.h_v * int64_t(P.dv) * 4);
  const int parts = cpr::backward_chunked_parts(P.dk);
  int64_t ws_bytes, bw_bytes;
  chunked_stash_parts(P, total_tokens, num_seqs, &ws_bytes, &bw_bytes);
  const char* st = static_cast<const char*>(stash);
  char* ws = static_cast<char*>(workspace);
  cpr::BackwardArgs A{};
  A.cu = cu_seqlens;
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b;
  A.d_o = d_o;
  A.d_state = d_state;
  A.chunk_states = chunk_states;
  A.fws = reinterpret_cast<const float*>(st);
  A.fbw = reinterpret_cast<const float*>(st + ws_bytes);
  A.cc = const_cast<float*>(A.fbw + rows * P.h_v * cpr::chunked_bwd_floats(P.dk));
  A.adjoint = reinterpret_cast<float*>(ws);
  A.dc = reinterpret_cast<float*>(ws + adj_bytes);
  A.ww = reinterpret_cast<float*>(ws + adj_bytes + tok_bytes);
  A.hpart = reinterpret_cast<double*>(ws + adj_bytes + 2 * tok_bytes);
  A.xv = reinterpret_cast<float*>(ws + adj_bytes + 2 * tok_bytes + align256((rows + num_seqs) * P.h_v * parts * 8));
  A.have_cw = 1;
  A.hparts = parts;
  A.dq = dq; A.dk = dk; A.dv = dv; A.da = da; A.db = db;
  A.d_state0 = d_state0;
  A.total_tokens = total_tokens;
  A.rows_cap = rows;
  A.adj_rows = rows + num_seqs;
  A.num_seqs = num_seqs;
  A.h_k = P.h_k; A.h_v = P.h_v; A.chunk = P.chunk;
  A.events = events;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = cpr::launch_backward_chunked(P.dk, A, hs);
  if (e != hipSuccess) return hip_fail(e, (std::string(fn) + " launch").c_str());
  e = cpr::launch_gradient_passes(P.dk, P.io_dtype, A, hs);
  if (e != hipSuccess) return hip_fail(e, (std::string(fn) + " gradient passes").c_str());
  return ok();
}

}  // extern "C"
