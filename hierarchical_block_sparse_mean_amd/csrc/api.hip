// C ABI of the PISA hot path: argument validation, pyramid geometry,
// workspace layout and kernel launches.  See include/pisa.h for the contract.
#include <math.h>
#include <string.h>

#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pisa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

pisa_status fail(pisa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pisa_status ok() {
  g_last_error.clear();
  return PISA_OK;
}

pisa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// product of non-negative int32 factors, exact (at most 2^124)
__int128 prod(std::initializer_list<int64_t> f) {
  __int128 r = 1;
  for (int64_t x : f) r *= x;
  return r;
}
// tensors far beyond any device memory: every element offset fits int64 below
constexpr int64_t kMaxTensorElems = (int64_t)1 << 46;

bool supported_group(int32_t G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

pisa::PyrGeom make_geom(int64_t cap, int32_t C) {
  pisa::PyrGeom g{};
  g.levels_cap = pisa::num_levels(cap, C);
  int64_t off = 0;
  for (int32_t l = 1; l <= g.levels_cap; ++l) {
    g.level_off[l] = off;
    off += pisa::level_rows(cap, C, l);
  }
  g.rows = off;
  return g;
}

// Validates a problem and fills the internal form.
pisa_status validate(const pisa_problem* p, pisa::Problem* out) {
  if (p == nullptr) return fail(PISA_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 1 || p->N < 1 || p->Hq < 1 || p->Hkv < 1 || p->D < 1)
    return fail(PISA_ERR_INVALID_ARG, "B, N, Hq, Hkv, D must be >= 1 (got %d %d %d %d %d)", p->B, p->N, p->Hq,
                p->Hkv, p->D);
  if (p->Hq % p->Hkv != 0) return fail(PISA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->C < 1) return fail(PISA_ERR_INVALID_ARG, "C must be >= 1 (got %d)", p->C);
  if (p->K < 1) return fail(PISA_ERR_INVALID_ARG, "K must be >= 1 (got %d)", p->K);
  if (p->causal != 0 && p->causal != 1) return fail(PISA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->dtype != PISA_F32 && p->dtype != PISA_BF16) return fail(PISA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return fail(PISA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (p->cap != 0 && p->cap < p->N) return fail(PISA_ERR_INVALID_ARG, "cap (%d) must be 0 or >= N (%d)", p->cap, p->N);
  if (p->select_algo < 0 || p->select_algo > 2) return fail(PISA_ERR_INVALID_ARG, "unknown select_algo %d", p->select_algo);
  if (p->attn_algo < 0 || p->attn_algo > 2) return fail(PISA_ERR_INVALID_ARG, "unknown attn_algo %d", p->attn_algo);
  if (p->q_tile < 0) return fail(PISA_ERR_INVALID_ARG, "q_tile must be >= 0");
  const int32_t G = p->Hq / p->Hkv;
  if (p->g != 2) return fail(PISA_ERR_UNSUPPORTED, "merge factor g must be 2 (got %d)", p->g);
  if (p->D != 64 && p->D != 128) return fail(PISA_ERR_UNSUPPORTED, "head dim D must be 64 or 128 (got %d)", p->D);
  if (!supported_group(G)) return fail(PISA_ERR_UNSUPPORTED, "G_Q = Hq/Hkv must be 1, 2, 4, 8 or 16 (got %d)", G);
  if (p->K > 32) return fail(PISA_ERR_UNSUPPORTED, "K must be <= 32 (got %d)", p->K);
  if (p->C > 128) return fail(PISA_ERR_UNSUPPORTED, "C must be <= 128 (got %d)", p->C);
  // stage-2 queries per key-fragment read: one 16-column tile (16/G_Q
  // queries) or two (32/G_Q: 16-bit inputs, C = 32, 64 or 128)
  const bool two_tiles = p->dtype == PISA_BF16 && (p->C == 32 || p->C == 64 || p->C == 128);
  if (p->q_tile != 0 && p->q_tile != 16 / G && !(two_tiles && p->q_tile == 32 / G))
    return fail(PISA_ERR_UNSUPPORTED, "q_tile must be 0, 16/G_Q = %d%s (got %d)", 16 / G,
                two_tiles ? " or 32/G_Q" : "", p->q_tile);
  const int64_t cap = p->cap ? p->cap : p->N;
  if (prod({p->B, p->Hkv, p->N, p->K}) > INT32_MAX) return fail(PISA_ERR_UNSUPPORTED, "B*Hkv*N*K exceeds 2^31-1");
  // (q and o stay below 2^42 elements by the bound above)
  if (prod({p->B, p->Hkv, cap, p->D}) >= kMaxTensorElems)
    return fail(PISA_ERR_UNSUPPORTED, "k and v (B*Hkv*cap*D) would exceed 2^46 elements");
  if (p->N >= (1 << 26)) return fail(PISA_ERR_UNSUPPORTED, "N must be < 2^26 (got %d)", p->N);
  out->B = p->B;
  out->N = p->N;
  out->Hq = p->Hq;
  out->Hkv = p->Hkv;
  out->G = G;
  out->D = p->D;
  out->C = p->C;
  out->K = p->K;
  out->causal = p->causal != 0;
  out->dtype = p->dtype;
  out->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D);
  out->cap = cap;
  out->L = pisa::num_levels(p->N, p->C);
  out->q_tile = p->q_tile ? p->q_tile : (two_tiles ? 32 / G : 16 / G);
  out->geo = make_geom(cap, p->C);
  // kernels address the rows of one head's summaries with 32-bit offsets
  if (out->geo.rows * (int64_t)p->D > INT32_MAX)
    return fail(PISA_ERR_UNSUPPORTED, "summary rows per head (%lld) x D (%d) must be < 2^31: cap / C is too large",
                (long long)out->geo.rows, p->D);
  return ok();
}

size_t blk2_bytes(const pisa::Problem& q) { return align256(sizeof(int32_t) * (size_t)q.B * q.Hkv * q.N * q.K); }

// ---- library-owned selection scratch (pisa_select_noalloc) ------------------
// One array per GPU, alive until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress with that
// device current) and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[PISA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
pisa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PISA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PISA_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(PISA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PISA_OK;
}

// pisa_select's work once its arguments are validated: stage 1 into the
// first part of ws, then stage 2 and the final top-K (or the fused program)
pisa_status run_select(const pisa::Problem& pr, int32_t algo, const void* q, const void* k, const float* pyr,
                       int32_t* idx, float* score, void* ws, hipStream_t stream) {
  if (algo == PISA_SELECT_FUSED)
    return hip_status(pisa::launch_route(pr, q, k, pyr, idx, score, true, stream), "pisa_select (fused)");
  int32_t* blk2 = static_cast<int32_t*>(ws);
  void* ws2 = static_cast<char*>(ws) + blk2_bytes(pr);
  hipError_t e = pisa::launch_route(pr, q, k, pyr, blk2, nullptr, false, stream);
  if (e != hipSuccess) return hip_status(e, "pisa_select (stage 1)");
  return hip_status(pisa::launch_stage2(pr, q, k, blk2, idx, score, ws2, stream), "pisa_select (stage 2)");
}

// ---- per-kernel timer ------------------------------------------------------
struct TimerRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_timer_mu;
bool g_timer_on = false;
std::vector<TimerRecord> g_records;
std::vector<hipEvent_t> g_event_pool;
hipEvent_t g_open_start = nullptr;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace pisa {
void timer_begin(const char* name, hipStream_t stream) {
  (void)name;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (!g_timer_on) return;
  g_open_start = take_event();
  if (g_open_start) hipEventRecord(g_open_start, stream);
}
void timer_end(const char* name, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (!g_timer_on || g_open_start == nullptr) return;
  hipEvent_t stop = take_event();
  if (stop == nullptr) return;
  hipEventRecord(stop, stream);
  g_records.push_back({name, g_open_start, stop});
  g_open_start = nullptr;
}
}  // namespace pisa

extern "C" {

void pisa_timer_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (auto& r : g_records) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  g_timer_on = on != 0;
}

int32_t pisa_timer_report(char* buf, size_t cap) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  std::map<std::string, std::pair<int64_t, double>> agg;
  for (auto& r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      auto& a = agg[r.name];
      a.first += 1;
      a.second += ms;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  std::string out;
  char line[256];
  for (auto& kv : agg) {
    snprintf(line, sizeof line, "%s\t%lld\t%.6f\n", kv.first.c_str(), (long long)kv.second.first, kv.second.second);
    out += line;
  }
  if (buf != nullptr && cap > 0) {
    const size_t n = out.size() < cap - 1 ? out.size() : cap - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return (int32_t)agg.size();
}

const char* pisa_last_error(void) { return g_last_error.c_str(); }

const char* pisa_version(void) { return "pisa-mi355x 0.1 (gfx950)"; }

int32_t pisa_levels(int64_t n, int32_t C) { return (n < 1 || C < 1) ? 0 : pisa::num_levels(n, C); }

int64_t pisa_level_rows(int64_t n, int32_t C, int32_t l) {
  if (n < 1 || C < 1 || l < 1 || l > 62) return 0;
  // a block spans C 2^(l-1) tokens, which can exceed 64 bits for levels far
  // above the top one (such a block holds all n tokens)
  const unsigned __int128 span = (unsigned __int128)C << (l - 1);
  const unsigned __int128 nn = (unsigned __int128)n;
  return span >= nn ? 1 : (int64_t)((nn + span - 1) / span);
}

int64_t pisa_level_offset(int64_t cap, int32_t C, int32_t l) {
  if (cap < 1 || C < 1 || l < 1 || l > pisa::num_levels(cap, C)) return -1;
  int64_t off = 0;
  for (int32_t i = 1; i < l; ++i) off += pisa::level_rows(cap, C, i);
  return off;
}

size_t pisa_pyramid_bytes(const pisa_problem* p) {
  pisa::Problem q;
  if (validate(p, &q) != PISA_OK) return 0;
  // fp32 rows, their fp16 block-floating-point copy, one int32 exponent per row
  return (size_t)q.B * q.Hkv * q.geo.rows * (q.D * (sizeof(float) + 2) + sizeof(int32_t));
}

pisa_status pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyr, hipStream_t stream) {
  pisa::Problem q;
  pisa_status s = validate(p, &q);
  if (s != PISA_OK) return s;
  if (k == nullptr || pyr == nullptr) return fail(PISA_ERR_INVALID_ARG, "k and pyr must be non-NULL");
  return hip_status(pisa::launch_build_pyramid(q, k, pyr, stream), "pisa_build_pyramid");
}

size_t pisa_select_workspace_bytes(const pisa_problem* p) {
  pisa::Problem q;
  if (validate(p, &q) != PISA_OK) return 0;
  if (p->select_algo == PISA_SELECT_FUSED) return 256;
  return blk2_bytes(q) + pisa::stage2_workspace_bytes(q);
}

pisa_status pisa_select(const pisa_problem* p, const void* q, const void* k, const float* pyr, int32_t* idx,
                        float* score, void* ws, size_t ws_bytes, hipStream_t stream) {
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (q == nullptr || k == nullptr || pyr == nullptr || idx == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, k, pyr and idx must be non-NULL");
  if (p->select_algo == PISA_SELECT_FUSED) return run_select(pr, p->select_algo, q, k, pyr, idx, score, nullptr, stream);
  const size_t need = blk2_bytes(pr) + pisa::stage2_workspace_bytes(pr);
  if (ws == nullptr || ws_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws == nullptr ? 0 : ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(PISA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return run_select(pr, p->select_algo, q, k, pyr, idx, score, ws, stream);
}

pisa_status pisa_select_noalloc(const pisa_problem* p, const void* q, const void* k, const float* pyr, int32_t* idx,
                                float* score, hipStream_t stream) {
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (q == nullptr || k == nullptr || pyr == nullptr || idx == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, k, pyr and idx must be non-NULL");
  const size_t need = p->select_algo == PISA_SELECT_FUSED ? 0 : blk2_bytes(pr) + pisa::stage2_workspace_bytes(pr);
  if (need > (size_t)PISA_NOALLOC_SCRATCH_BYTES)
    return fail(PISA_ERR_WORKSPACE,
                "pisa_select_noalloc: this problem needs %zu bytes of scratch, beyond the library's %zu; "
                "call pisa_select with a workspace instead",
                need, (size_t)PISA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    s = scratch_address(&ws);
    if (s != PISA_OK) return s;
  }
  return run_select(pr, p->select_algo, q, k, pyr, idx, score, ws, stream);
}

pisa_status pisa_route_counts(const pisa_problem* p, const void* q, const void* k, const float* pyr,
                              uint64_t* counts, void* ws, size_t ws_bytes, hipStream_t stream) {
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (q == nullptr || k == nullptr || pyr == nullptr || counts == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, k, pyr and counts must be non-NULL");
  if (pr.dtype != PISA_BF16) return fail(PISA_ERR_UNSUPPORTED, "work counters exist for the bf16 stage-1 kernel only");
  if (ws == nullptr || ws_bytes < blk2_bytes(pr))
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed", blk2_bytes(pr));
  return hip_status(pisa::launch_route(pr, q, k, pyr, static_cast<int32_t*>(ws), nullptr, false, stream,
                                       reinterpret_cast<unsigned long long*>(counts)),
                    "pisa_route_counts");
}

size_t pisa_attn_workspace_bytes(const pisa_problem* p) {
  pisa::Problem q;
  if (validate(p, &q) != PISA_OK) return 0;
  if (p->attn_algo == PISA_ATTN_QUERY_MAJOR) return 256;
  return pisa::attn_leaf_workspace_bytes(q);
}

pisa_status pisa_sparse_attn(const pisa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                             void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || idx == nullptr || o == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, k, v, idx and o must be non-NULL");
  if (p->attn_algo == PISA_ATTN_QUERY_MAJOR)
    return hip_status(pisa::launch_attn_query(pr, q, k, v, idx, o, lse, stream), "pisa_sparse_attn (query-major)");
  const size_t need = pisa::attn_leaf_workspace_bytes(pr);
  if (ws == nullptr || ws_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws == nullptr ? 0 : ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(PISA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(pisa::launch_attn_leaf(pr, q, k, v, idx, o, lse, ws, stream), "pisa_sparse_attn (leaf-major)");
}

// fp32 rows of d = 128 with C > 64: a leaf's K, V and K^T tiles exceed the LDS
static bool bwd_shape_unsupported(const pisa::Problem& q) { return q.dtype == 0 && q.D == 128 && q.C > 64; }

size_t pisa_attn_backward_workspace_bytes(const pisa_problem* p) {
  pisa::Problem q;
  if (validate(p, &q) != PISA_OK || bwd_shape_unsupported(q)) return 0;
  return pisa::attn_bwd_workspace_bytes(q);
}

pisa_status pisa_sparse_attn_backward(const pisa_problem* p, const void* q, const void* k, const void* v,
                                      const int32_t* idx, const void* o, const float* lse, const void* dout,
                                      void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (bwd_shape_unsupported(pr))
    return fail(PISA_ERR_UNSUPPORTED, "backward with fp32 rows of d = 128 needs C <= 64 (got C = %d)", pr.C);
  if (q == nullptr || k == nullptr || v == nullptr || idx == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, k, v, idx, o, lse, dout, dq, dk and dv must be non-NULL");
  const size_t need = pisa::attn_bwd_workspace_bytes(pr);
  if (ws == nullptr || ws_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws == nullptr ? 0 : ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(PISA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(pisa::launch_attn_bwd(pr, q, k, v, idx, o, lse, dout, dq, dk, dv, ws, stream),
                    "pisa_sparse_attn_backward");
}

size_t pisa_flat_workspace_bytes(const pisa_problem* p) {
  pisa::Problem q;
  if (validate(p, &q) != PISA_OK) return 0;
  return 256;
}

pisa_status pisa_flat_select(const pisa_problem* p, const void* q, const float* pyr, int32_t* idx, float* score,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  pisa::Problem pr;
  pisa_status s = validate(p, &pr);
  if (s != PISA_OK) return s;
  if (q == nullptr || pyr == nullptr || idx == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "q, pyr and idx must be non-NULL");
  return hip_status(pisa::launch_flat(pr, q, pyr, idx, score, stream), "pisa_flat_select");
}

pisa_status pisa_decode_step(const pisa_decode_problem* p, void* k_cache, void* v_cache, float* pyr, int32_t* len,
                             const void* q_new, const void* k_new, const void* v_new, void* o, int32_t* idx,
                             float* score, int32_t* err, hipStream_t stream) {
  if (p == nullptr) return fail(PISA_ERR_INVALID_ARG, "problem is NULL");
  if (p->S < 1 || p->cap < 1 || p->Hq < 1 || p->Hkv < 1 || p->D < 1 || p->C < 1 || p->K < 1)
    return fail(PISA_ERR_INVALID_ARG, "S, cap, Hq, Hkv, D, C, K must be >= 1");
  if (p->Hq % p->Hkv != 0) return fail(PISA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->dtype != PISA_F32 && p->dtype != PISA_BF16) return fail(PISA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return fail(PISA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  const int32_t G = p->Hq / p->Hkv;
  if (p->g != 2) return fail(PISA_ERR_UNSUPPORTED, "merge factor g must be 2 (got %d)", p->g);
  if (p->D != 64 && p->D != 128) return fail(PISA_ERR_UNSUPPORTED, "head dim D must be 64 or 128 (got %d)", p->D);
  if (!supported_group(G)) return fail(PISA_ERR_UNSUPPORTED, "G_Q = Hq/Hkv must be 1, 2, 4, 8 or 16 (got %d)", G);
  if (p->K > 32) return fail(PISA_ERR_UNSUPPORTED, "K must be <= 32 (got %d)", p->K);
  if (p->C > 128) return fail(PISA_ERR_UNSUPPORTED, "C must be <= 128 (got %d)", p->C);
  if (prod({p->S, p->Hkv, p->cap, p->D}) >= kMaxTensorElems || prod({p->S, p->Hq, p->D}) >= kMaxTensorElems)
    return fail(PISA_ERR_UNSUPPORTED, "the caches would exceed 2^46 elements");
  if (k_cache == nullptr || v_cache == nullptr || pyr == nullptr || len == nullptr || q_new == nullptr ||
      k_new == nullptr || v_new == nullptr || o == nullptr)
    return fail(PISA_ERR_INVALID_ARG, "k_cache, v_cache, pyr, len, q_new, k_new, v_new and o must be non-NULL");
  pisa::DecodeArgs a{};
  a.S = p->S;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = G;
  a.D = p->D;
  a.C = p->C;
  a.K = p->K;
  a.dtype = p->dtype;
  a.cap = p->cap;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D);
  a.geo = make_geom(p->cap, p->C);
  return hip_status(pisa::launch_decode(a, k_cache, v_cache, pyr, len, q_new, k_new, v_new, o, idx, score, err, stream),
                    "pisa_decode_step");
}

}  // extern "C"
