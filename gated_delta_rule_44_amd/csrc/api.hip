// api.hip -- the C ABI declared in include/gdr.h: host-side argument checks,
// dispatch over dtype x gate x width, and launches on the caller's stream.
// Every check runs before the first HIP call, so a rejected call has no side
// effects.  No C++ exception crosses the interface.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/gdr.h"
#include "gdr_internal.h"

namespace {

thread_local char g_err[512] = "";

gdr_status fail(gdr_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

bool debug_sync() {
    static const int on = [] {
        const char *e = getenv("GDR_DEBUG");
        return (e && e[0] && e[0] != '0') ? 1 : 0;
    }();
    return on != 0;
}

gdr_status finish(hipError_t launch, hipStream_t s, const char *what) {
    if (launch != hipSuccess)
        return fail(GDR_EHIP, "%s: launch failed: %s", what, hipGetErrorString(launch));
    if (debug_sync()) {
        hipError_t e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess)
            return fail(GDR_EHIP, "%s: execution failed: %s", what, hipGetErrorString(e));
    }
    return GDR_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// (sequence, head) pairs of one prefill call: the prefill kernels launch up
// to four workgroups per pair, rounded up to eight pairs, in a 31-bit grid
constexpr long long kMaxPairs = 1LL << 28;

gdr_status check_common(int dt, int gk, int Dk, int Dv, const char *what) {
    if (dt != GDR_F32 && dt != GDR_BF16)
        return fail(GDR_EINVAL, "%s: dtype %d is not GDR_F32 or GDR_BF16", what, dt);
    if (gk != GDR_GATE_SCALAR && gk != GDR_GATE_CHANNEL)
        return fail(GDR_EINVAL, "%s: gate kind %d is not scalar or channel", what, gk);
    if (Dk != Dv)
        return fail(GDR_EUNSUPPORTED, "%s: Dk (%d) != Dv (%d) is not supported", what, Dk, Dv);
    if (Dk != 64 && Dk != 128)
        return fail(GDR_EUNSUPPORTED, "%s: Dk = %d; supported widths are 64 and 128", what, Dk);
    return GDR_OK;
}

#define REQUIRE_PTR(p, name)                                                        \
    do {                                                                            \
        if (!(p)) return fail(GDR_EINVAL, "%s: %s is NULL", what, name);            \
        if (!aligned16(p)) return fail(GDR_EINVAL, "%s: %s is not 16-byte aligned", \
                                       what, name);                                 \
    } while (0)
#define REQUIRE_ALIGNED_OR_NULL(p, name)                                            \
    do {                                                                            \
        if ((p) && !aligned16(p)) return fail(GDR_EINVAL,                           \
                                              "%s: %s is not 16-byte aligned",      \
                                              what, name);                          \
    } while (0)

gdr_status check_prefill_ptrs(const char *what, const void *q, const void *k, const void *v,
                              const void *g, const void *beta, const float *h0,
                              const void *o, const float *ht, long long tokens) {
    if (tokens > 0) {
        REQUIRE_PTR(q, "q");
        REQUIRE_PTR(k, "k");
        REQUIRE_PTR(v, "v");
        REQUIRE_PTR(g, "g");
        if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
        REQUIRE_PTR(o, "o");
    }
    REQUIRE_ALIGNED_OR_NULL(h0, "h0");
    REQUIRE_ALIGNED_OR_NULL(ht, "ht");
    return GDR_OK;
}

gdr_status check_workspace(const char *what, const void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return GDR_OK;
    if (!ws || ws_bytes < need)
        return fail(GDR_EINVAL, "%s: workspace of %zu bytes needed, %zu given", what, need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(GDR_EINVAL, "%s: workspace is not 16-byte aligned", what);
    return GDR_OK;
}

// Workspace of one prefill call: the varlen schedule (N int32), the first
// chunk of each packed sequence (N+1 int32), for the bf16 channel-gate path
// one int32 per (sequence, head) (the pairs the plain pass leaves to the
// reference pass) and, for the bf16 scalar-gate path, one kTileBytes
// record per (chunk, head).  Chunk records are counted as tokens / 64 + N,
// which bounds sum_n ceil(len_n / 64).
struct WsLayout {
    size_t order, chunk_base, units, tiles, total;
    long long max_chunks;
};
WsLayout ws_layout(bool tiles, bool units, int N, long long tokens, int H,
                   size_t rec = gdr::kTileBytes) {
    WsLayout w{};
    if (N <= 0 || tokens < 0 || H <= 0) return w;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    w.order = 0;
    w.chunk_base = r256((size_t)N * sizeof(int32_t));
    w.units = w.chunk_base + r256((size_t)(N + 1) * sizeof(int32_t));
    w.tiles = w.units + (units ? r256((size_t)N * H * sizeof(int32_t)) : 0);
    w.max_chunks = tiles ? tokens / 64 + N : 0;
    w.total = w.tiles + (size_t)w.max_chunks * H * rec;
    return w;
}
// the layout of a prefill call in dtype dt with gate kind gk
WsLayout prefill_layout(int dt, int gk, int N, long long tokens, int H, bool raw) {
    return ws_layout(dt == GDR_BF16 && gk == GDR_GATE_SCALAR, dt == GDR_BF16 && gk == GDR_GATE_CHANNEL,
                     N, tokens, H, raw ? gdr::kTileBytesRaw : gdr::kTileBytes);
}

// packed-batch prefill shared by the plain and the pool entry points
// g and beta: fp32 gate logs and write strengths, or (raw) logits in dt
gdr_status prefill_varlen_impl(const char *what, int dt, int gk, int N, int T_total, int H,
                               int Dk, int Dv, int chunk, float scale,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               const void *q, const void *k, const void *v, const void *g,
                               const void *beta, bool raw, float gate_scale, const float *h0,
                               void *o, float *ht, const int32_t *h0_slot,
                               const int32_t *ht_slot, long long pool, void *workspace,
                               size_t ws_bytes, void *stream);
gdr_status prefill_fixed_impl(const char *what, int dt, int gk, int B, int T, int H, int Dk,
                              int Dv, int chunk, float scale, const void *q, const void *k,
                              const void *v, const void *g, const void *beta, bool raw,
                              float gate_scale, const float *h0, void *o, float *ht,
                              void *workspace, size_t ws_bytes, void *stream);

gdr_status check_gate_scale(const char *what, float c) {
    if (!(c >= 0.f))   // also rejects NaN
        return fail(GDR_EINVAL, "%s: gate_scale = %g; it must be >= 0", what, (double)c);
    return GDR_OK;
}

}  // namespace

extern "C" {

const char *gdr_last_error(void) { return g_err; }

const char *gdr_version(void) { return "gdr 0.1.0 (gfx950)"; }

size_t gdr_prefill_workspace_bytes(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                   long long tokens, int H) {
    return prefill_layout(dt, gk, N, tokens, H, false).total;
}

size_t gdr_prefill_fused_workspace_bytes(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                         long long tokens, int H) {
    return prefill_layout(dt, gk, N, tokens, H, true).total;
}

gdr_status gdr_prefill_chunked(enum gdr_dtype dt, enum gdr_gate gk, int B, int T, int H,
                               int Dk, int Dv, int chunk, float scale, const void *q,
                               const void *k, const void *v, const float *g,
                               const float *beta, const float *h0, void *o, float *ht,
                               void *workspace, size_t ws_bytes, void *stream) {
    return prefill_fixed_impl("gdr_prefill_chunked", dt, gk, B, T, H, Dk, Dv, chunk, scale, q, k,
                              v, g, beta, false, 0.f, h0, o, ht, workspace, ws_bytes, stream);
}

gdr_status gdr_prefill_chunked_fused(enum gdr_dtype dt, enum gdr_gate gk, int B, int T, int H,
                                     int Dk, int Dv, int chunk, float scale, const void *q,
                                     const void *k, const void *v, const void *gate_logit,
                                     const void *beta_logit, float gate_scale, const float *h0,
                                     void *o, float *ht, void *workspace, size_t ws_bytes,
                                     void *stream) {
    const char *what = "gdr_prefill_chunked_fused";
    gdr_status st = check_gate_scale(what, gate_scale);
    if (st != GDR_OK) return st;
    return prefill_fixed_impl(what, dt, gk, B, T, H, Dk, Dv, chunk, scale, q, k, v, gate_logit,
                              beta_logit, true, gate_scale, h0, o, ht, workspace, ws_bytes,
                              stream);
}

}  // extern "C"

namespace {

gdr_status prefill_fixed_impl(const char *what, int dt, int gk, int B, int T, int H, int Dk,
                              int Dv, int chunk, float scale, const void *q, const void *k,
                              const void *v, const void *g, const void *beta, bool raw,
                              float gate_scale, const float *h0, void *o, float *ht,
                              void *workspace, size_t ws_bytes, void *stream) {
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (chunk != 64) return fail(GDR_EUNSUPPORTED, "%s: chunk = %d; only 64 is supported", what, chunk);
    if (B < 0 || T < 0 || H <= 0)
        return fail(GDR_EINVAL, "%s: bad sizes B=%d T=%d H=%d", what, B, T, H);
    if ((long long)B * T * H * Dk >= (1LL << 40))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    // one workgroup per (sequence, head, value slice): the grid must stay a
    // 31-bit count (with the bound above, so does the number of chunk records)
    if ((long long)B * H > kMaxPairs)
        return fail(GDR_EUNSUPPORTED, "%s: %lld (sequence, head) pairs exceed %lld", what,
                    (long long)B * H, kMaxPairs);
    st = check_prefill_ptrs(what, q, k, v, g, beta, h0, o, ht, (long long)B * T);
    if (st != GDR_OK) return st;
    if (h0 && ht && h0 != ht) {
        const size_t bytes = (size_t)B * H * Dv * Dk * sizeof(float);
        const char *a0 = (const char *)h0, *a1 = (const char *)ht;
        if (a0 < a1 + bytes && a1 < a0 + bytes)
            return fail(GDR_EINVAL, "%s: h0 and ht overlap without being equal", what);
    }
    if (B == 0) return GDR_OK;
    const bool tiles = dt == GDR_BF16 && gk == GDR_GATE_SCALAR;
    const bool units = dt == GDR_BF16 && gk == GDR_GATE_CHANNEL;
    const WsLayout L = prefill_layout(dt, gk, B, (long long)B * T, H, raw);
    st = check_workspace(what, workspace, ws_bytes, tiles || units ? L.total : 0);
    if (st != GDR_OK) return st;
    gdr::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.h0 = h0; a.o = o; a.ht = ht;
    if (raw) {
        a.xg = g; a.xb = beta; a.gate_scale = gate_scale;
    } else {
        a.g = static_cast<const float *>(g); a.beta = static_cast<const float *>(beta);
    }
    a.cu_seqlens = nullptr; a.order = nullptr; a.chunk_base = nullptr;
    a.tiles = tiles ? static_cast<char *>(workspace) + L.tiles : nullptr;
    a.unit_wide = units ? reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + L.units) : nullptr;
    a.max_chunks = tiles ? (long long)B * ((T + 63) / 64) : 0;
    a.N = B; a.T = T; a.H = H; a.scale = scale; a.channel_gate = gk == GDR_GATE_CHANNEL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dt == GDR_BF16 ? gdr::launch_prefill_chunked(Dk, a, s)
                                  : gdr::launch_prefill_recurrent(false, Dk, a, s);
    return finish(e, s, what);
}

// The library's own workspace for gdr_prefill_chunked_noalloc: one array per
// GPU, held from the library's first use on that GPU until the process
// ends.  Host code never passes the array's name to a kernel (in host code
// it names a host-side stand-in); it passes the device address that
// hipGetSymbolAddress returns, taken once per device with that device
// current.
constexpr size_t kScratchBytes = GDR_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

gdr_status scratch_of_current_device(const char *what, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GDR_EHIP, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDR_EUNSUPPORTED, "%s: device %d is beyond the %d the library tracks", what,
                    dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GDR_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d failed: %s",
                        what, dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_prefill_chunked_noalloc(enum gdr_dtype dt, enum gdr_gate gk, int B, int T, int H,
                                       int Dk, int Dv, int chunk, float scale, const void *q,
                                       const void *k, const void *v, const float *g,
                                       const float *beta, const float *h0, void *o, float *ht,
                                       void *stream) {
    const char *what = "gdr_prefill_chunked_noalloc";
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (B < 0 || T < 0 || H <= 0)
        return fail(GDR_EINVAL, "%s: bad sizes B=%d T=%d H=%d", what, B, T, H);
    const size_t need = prefill_layout(dt, gk, B, (long long)B * T, H, false).total;
    if (need > kScratchBytes)
        return fail(GDR_EUNSUPPORTED,
                    "%s: this call needs %zu bytes of workspace, beyond the library's own %zu "
                    "(use gdr_prefill_chunked with a workspace of that size)",
                    what, need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_of_current_device(what, &ws);
        if (st != GDR_OK) return st;
    }
    return prefill_fixed_impl(what, dt, gk, B, T, H, Dk, Dv, chunk, scale, q, k, v, g, beta,
                              false, 0.f, h0, o, ht, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"

extern "C" {

gdr_status gdr_prefill_chunked_varlen(enum gdr_dtype dt, enum gdr_gate gk, int N, int T_total,
                                      int H, int Dk, int Dv, int chunk, float scale,
                                      const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                      const void *q, const void *k, const void *v,
                                      const float *g, const float *beta, const float *h0,
                                      void *o, float *ht, void *workspace, size_t ws_bytes,
                                      void *stream) {
    const char *what = "gdr_prefill_chunked_varlen";
    if (h0 && ht && h0 != ht && N > 0 && H > 0 && Dk > 0 && Dv > 0) {
        const size_t bytes = (size_t)N * H * Dv * Dk * sizeof(float);
        const char *a0 = (const char *)h0, *a1 = (const char *)ht;
        if (a0 < a1 + bytes && a1 < a0 + bytes)
            return fail(GDR_EINVAL, "%s: h0 and ht overlap without being equal", what);
    }
    return prefill_varlen_impl(what, dt, gk, N, T_total, H, Dk, Dv, chunk, scale, cu_seqlens,
                               cu_seqlens_host, q, k, v, g, beta, false, 0.f, h0, o, ht,
                               nullptr, nullptr, 0, workspace, ws_bytes, stream);
}

gdr_status gdr_prefill_varlen_fused(enum gdr_dtype dt, enum gdr_gate gk, int N, int T_total,
                                    int H, int Dk, int Dv, int chunk, float scale,
                                    const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                    const void *q, const void *k, const void *v,
                                    const void *gate_logit, const void *beta_logit,
                                    float gate_scale, const float *h0, void *o, float *ht,
                                    void *workspace, size_t ws_bytes, void *stream) {
    const char *what = "gdr_prefill_varlen_fused";
    gdr_status st = check_gate_scale(what, gate_scale);
    if (st != GDR_OK) return st;
    if (h0 && ht && h0 != ht && N > 0 && H > 0 && Dk > 0 && Dv > 0) {
        const size_t bytes = (size_t)N * H * Dv * Dk * sizeof(float);
        const char *a0 = (const char *)h0, *a1 = (const char *)ht;
        if (a0 < a1 + bytes && a1 < a0 + bytes)
            return fail(GDR_EINVAL, "%s: h0 and ht overlap without being equal", what);
    }
    return prefill_varlen_impl(what, dt, gk, N, T_total, H, Dk, Dv, chunk, scale, cu_seqlens,
                               cu_seqlens_host, q, k, v, gate_logit, beta_logit, true,
                               gate_scale, h0, o, ht, nullptr, nullptr, 0, workspace, ws_bytes,
                               stream);
}

}  // extern "C"

namespace {

gdr_status prefill_varlen_impl(const char *what, int dt, int gk, int N, int T_total, int H,
                               int Dk, int Dv, int chunk, float scale,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               const void *q, const void *k, const void *v, const void *g,
                               const void *beta, bool raw, float gate_scale, const float *h0,
                               void *o, float *ht, const int32_t *h0_slot,
                               const int32_t *ht_slot, long long pool, void *workspace,
                               size_t ws_bytes, void *stream) {
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (chunk != 64) return fail(GDR_EUNSUPPORTED, "%s: chunk = %d; only 64 is supported", what, chunk);
    if (N < 0 || T_total < 0 || H <= 0)
        return fail(GDR_EINVAL, "%s: bad sizes N=%d T_total=%d H=%d", what, N, T_total, H);
    if ((long long)T_total * H * Dk >= (1LL << 40))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    if ((long long)N * H > kMaxPairs)
        return fail(GDR_EUNSUPPORTED, "%s: %lld (sequence, head) pairs exceed %lld", what,
                    (long long)N * H, kMaxPairs);
    if (N == 0) return GDR_OK;
    if (!cu_seqlens) return fail(GDR_EINVAL, "%s: cu_seqlens is NULL", what);
    if (cu_seqlens_host) {
        if (cu_seqlens_host[0] != 0)
            return fail(GDR_EINVAL, "%s: cu_seqlens[0] = %d, expected 0", what, cu_seqlens_host[0]);
        for (int i = 0; i < N; ++i)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
                return fail(GDR_EINVAL, "%s: cu_seqlens decreases at %d", what, i);
        if (cu_seqlens_host[N] != T_total)
            return fail(GDR_EINVAL, "%s: cu_seqlens[N] = %d but T_total = %d", what,
                        cu_seqlens_host[N], T_total);
    }
    st = check_prefill_ptrs(what, q, k, v, g, beta, h0, o, ht, T_total);
    if (st != GDR_OK) return st;
    const bool tiles = dt == GDR_BF16 && gk == GDR_GATE_SCALAR;
    const bool units = dt == GDR_BF16 && gk == GDR_GATE_CHANNEL;
    const WsLayout L = prefill_layout(dt, gk, N, T_total, H, raw);
    st = check_workspace(what, workspace, ws_bytes, L.total);
    if (st != GDR_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    int32_t *order = reinterpret_cast<int32_t *>(ws + L.order);
    hipError_t e = gdr::launch_varlen_schedule(cu_seqlens, N, order, s);
    if (e != hipSuccess) return finish(e, s, what);
    gdr::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.h0 = h0; a.o = o; a.ht = ht;
    if (raw) {
        a.xg = g; a.xb = beta; a.gate_scale = gate_scale;
    } else {
        a.g = static_cast<const float *>(g); a.beta = static_cast<const float *>(beta);
    }
    a.cu_seqlens = cu_seqlens; a.order = order;
    a.chunk_base = reinterpret_cast<int32_t *>(ws + L.chunk_base);
    a.tiles = tiles ? ws + L.tiles : nullptr;
    a.unit_wide = units ? reinterpret_cast<int32_t *>(ws + L.units) : nullptr;
    a.max_chunks = L.max_chunks;
    a.N = N; a.T = 0; a.H = H; a.scale = scale; a.channel_gate = gk == GDR_GATE_CHANNEL;
    a.h0_slot = h0_slot; a.ht_slot = ht_slot; a.pool = pool;
    e = dt == GDR_BF16 ? gdr::launch_prefill_chunked(Dk, a, s)
                       : gdr::launch_prefill_recurrent(false, Dk, a, s);
    return finish(e, s, what);
}

}  // namespace

extern "C" {


gdr_status gdr_prefill_varlen_pool(enum gdr_dtype dt, enum gdr_gate gk, int N, int T_total,
                                   int H, int Dk, int Dv, int chunk, float scale,
                                   const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                   const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, int pool_slots,
                                   float *state_pool, const int32_t *h0_slot,
                                   const int32_t *ht_slot, const int32_t *h0_slot_host,
                                   const int32_t *ht_slot_host, void *o, void *workspace,
                                   size_t ws_bytes, void *stream) {
    const char *what = "gdr_prefill_varlen_pool";
    if (pool_slots < 0) return fail(GDR_EINVAL, "%s: pool_slots = %d", what, pool_slots);
    if (N > 0) {
        if (!h0_slot || !ht_slot) return fail(GDR_EINVAL, "%s: h0_slot and ht_slot are required", what);
        REQUIRE_PTR(state_pool, "state_pool");
        if ((long long)pool_slots * H >= (1LL << 31))
            return fail(GDR_EUNSUPPORTED, "%s: pool of %d slots x %d heads too large", what,
                        pool_slots, H);
    }
    if (h0_slot_host && ht_slot_host && N > 0) {
        for (int n = 0; n < N; ++n) {
            if (h0_slot_host[n] < -1 || h0_slot_host[n] >= pool_slots)
                return fail(GDR_EINVAL, "%s: h0_slot[%d] = %d outside -1..%d", what, n,
                            h0_slot_host[n], pool_slots - 1);
            if (ht_slot_host[n] < -1 || ht_slot_host[n] >= pool_slots)
                return fail(GDR_EINVAL, "%s: ht_slot[%d] = %d outside -1..%d", what, n,
                            ht_slot_host[n], pool_slots - 1);
        }
        // a slot written by one sequence is neither written nor read by another
        for (int n = 0; n < N; ++n) {
            const int s = ht_slot_host[n];
            if (s < 0) continue;
            for (int m = 0; m < N; ++m) {
                if (m == n) continue;
                if (ht_slot_host[m] == s)
                    return fail(GDR_EINVAL, "%s: sequences %d and %d both write slot %d", what,
                                n, m, s);
                if (h0_slot_host[m] == s)
                    return fail(GDR_EINVAL, "%s: sequence %d reads slot %d that sequence %d writes",
                                what, m, s, n);
            }
        }
    }
    return prefill_varlen_impl(what, dt, gk, N, T_total, H, Dk, Dv, chunk, scale, cu_seqlens,
                               cu_seqlens_host, q, k, v, g, beta, false, 0.f, state_pool, o,
                               state_pool, h0_slot, ht_slot, pool_slots, workspace, ws_bytes,
                               stream);
}

gdr_status gdr_decode_step(enum gdr_dtype dt, enum gdr_gate gk, int B, int H, int Dk, int Dv,
                           float scale, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state, void *o,
                           void *stream) {
    const char *what = "gdr_decode_step";
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (B < 0 || H <= 0) return fail(GDR_EINVAL, "%s: bad sizes B=%d H=%d", what, B, H);
    if ((long long)B * H >= (1LL << 31))
        return fail(GDR_EUNSUPPORTED, "%s: B*H too large", what);
    if (B == 0) return GDR_OK;
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(g, "g");
    if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
    REQUIRE_PTR(state, "state");
    if (!o) return fail(GDR_EINVAL, "%s: o is NULL", what);
    gdr::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.B = B; a.H = H; a.scale = scale;
    a.g_bh = gk == GDR_GATE_CHANNEL ? Dk : 1;
    a.g_layer = 0;
    gdr::DecodeLayers layers;
    layers.n = 1;
    layers.code[0] = (uint16_t)(gk == GDR_GATE_CHANNEL ? 1 : 0);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdr::launch_decode(dt == GDR_BF16, Dk, a, layers, s), s, what);
}

gdr_status gdr_decode_placement(const uint8_t *placement, int L, enum gdr_dtype dt, int B,
                                int H, int Dk, int Dv, float scale, const void *q,
                                const void *k, const void *v, const float *g,
                                const float *beta, float *state_pool, void *o, void *stream) {
    const char *what = "gdr_decode_placement";
    gdr_status st = check_common(dt, GDR_GATE_CHANNEL, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (!placement) return fail(GDR_EINVAL, "%s: placement is NULL", what);
    if (L <= 0 || L > gdr::kMaxLayers)
        return fail(GDR_EINVAL, "%s: L = %d outside 1..%d", what, L, gdr::kMaxLayers);
    if (B < 0 || H <= 0) return fail(GDR_EINVAL, "%s: bad sizes B=%d H=%d", what, B, H);
    gdr::DecodeLayers layers;
    layers.n = 0;
    for (int l = 0; l < L; ++l) {
        const int c = placement[l];
        if (c > GDR_KDA)
            return fail(GDR_EINVAL, "%s: placement[%d] = %d is not a mixer code 0..3", what, l, c);
        if (c == GDR_GDN || c == GDR_KDA)
            layers.code[layers.n++] = (uint16_t)((l << 1) | (c == GDR_KDA ? 1 : 0));
    }
    if ((long long)layers.n * B * H >= (1LL << 31))
        return fail(GDR_EUNSUPPORTED, "%s: too many (layer, b, h) slots", what);
    if (B == 0 || layers.n == 0) return GDR_OK;
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(g, "g");
    if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
    REQUIRE_PTR(state_pool, "state_pool");
    if (!o) return fail(GDR_EINVAL, "%s: o is NULL", what);
    gdr::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state_pool; a.o = o;
    a.B = B; a.H = H; a.scale = scale;
    a.g_bh = Dk;
    a.g_layer = (long long)B * H * Dk;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdr::launch_decode(dt == GDR_BF16, Dk, a, layers, s), s, what);
}

}  // extern "C"

namespace {

// g and beta are fp32 gate logs and write strengths, or (raw) logits in dt
gdr_status decode_tokens_impl(const char *what, int dt, int gk, int B, int n_tok, int H,
                              int Dk, int Dv, float scale, const void *q, const void *k,
                              const void *v, const void *g, const void *beta, bool raw,
                              float gate_scale, const int32_t *slot, const int32_t *slot_host,
                              int pool_slots, float *state_pool, float *checkpoints, void *o,
                              void *stream) {
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (B < 0 || n_tok < 0 || H <= 0 || pool_slots < 0)
        return fail(GDR_EINVAL, "%s: bad sizes B=%d n_tok=%d H=%d pool_slots=%d", what, B,
                    n_tok, H, pool_slots);
    if ((long long)B * H >= (1LL << 27) || (long long)pool_slots * H >= (1LL << 31) ||
        (long long)B * n_tok * H * Dk >= (1LL << 40))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    if (!slot && pool_slots < B)
        return fail(GDR_EINVAL, "%s: without a slot map the pool needs B = %d slots, has %d",
                    what, B, pool_slots);
    if (slot_host) {
        if (!slot) return fail(GDR_EINVAL, "%s: slot_host given without slot", what);
        for (int b = 0; b < B; ++b)
            if (slot_host[b] < -1 || slot_host[b] >= pool_slots)
                return fail(GDR_EINVAL, "%s: slot[%d] = %d outside -1..%d", what, b,
                            slot_host[b], pool_slots - 1);
        // two sequences on one slot would race; sort a copy to find repeats
        int32_t *tmp = static_cast<int32_t *>(malloc(sizeof(int32_t) * (B > 0 ? B : 1)));
        if (!tmp) return fail(GDR_EINVAL, "%s: host memory for the slot check", what);
        memcpy(tmp, slot_host, sizeof(int32_t) * B);
        qsort(tmp, B, sizeof(int32_t), [](const void *x, const void *y) {
            const int32_t a = *static_cast<const int32_t *>(x), b = *static_cast<const int32_t *>(y);
            return (a > b) - (a < b);
        });
        int dup = -1;
        for (int b = 1; b < B && dup < 0; ++b)
            if (tmp[b] >= 0 && tmp[b] == tmp[b - 1]) dup = tmp[b];
        free(tmp);
        if (dup >= 0) return fail(GDR_EINVAL, "%s: slot %d is used by two sequences", what, dup);
    }
    if (B == 0 || n_tok == 0) return GDR_OK;
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(g, "g");
    if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
    REQUIRE_PTR(state_pool, "state_pool");
    REQUIRE_ALIGNED_OR_NULL(checkpoints, "checkpoints");
    if (!o) return fail(GDR_EINVAL, "%s: o is NULL", what);
    if (checkpoints) {
        const size_t pb = (size_t)pool_slots * H * Dv * Dk * sizeof(float);
        const size_t cb = (size_t)B * n_tok * H * Dv * Dk * sizeof(float);
        const char *p0 = (const char *)state_pool, *c0 = (const char *)checkpoints;
        if (p0 < c0 + cb && c0 < p0 + pb)
            return fail(GDR_EINVAL, "%s: checkpoints overlap state_pool", what);
    }
    gdr::TokensArgs a{};
    a.q = q; a.k = k; a.v = v;
    if (raw) {
        a.xg = g; a.xb = beta; a.gate_scale = gate_scale;
    } else {
        a.g = static_cast<const float *>(g); a.beta = static_cast<const float *>(beta);
    }
    a.slot = slot; a.pool = pool_slots; a.state = state_pool; a.ckpt = checkpoints; a.o = o;
    a.B = B; a.n = n_tok; a.H = H; a.scale = scale; a.channel_gate = gk == GDR_GATE_CHANNEL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdr::launch_decode_tokens(dt == GDR_BF16, Dk, a, s, raw), s, what);
}

}  // namespace

extern "C" {

gdr_status gdr_decode_tokens(enum gdr_dtype dt, enum gdr_gate gk, int B, int n_tok, int H,
                             int Dk, int Dv, float scale, const void *q, const void *k,
                             const void *v, const float *g, const float *beta,
                             const int32_t *slot, const int32_t *slot_host, int pool_slots,
                             float *state_pool, float *checkpoints, void *o, void *stream) {
    return decode_tokens_impl("gdr_decode_tokens", dt, gk, B, n_tok, H, Dk, Dv, scale, q, k, v,
                              g, beta, false, 0.f, slot, slot_host, pool_slots, state_pool,
                              checkpoints, o, stream);
}

gdr_status gdr_decode_tokens_fused(enum gdr_dtype dt, enum gdr_gate gk, int B, int n_tok,
                                   int H, int Dk, int Dv, float scale, const void *q,
                                   const void *k, const void *v, const void *gate_logit,
                                   const void *beta_logit, float gate_scale,
                                   const int32_t *slot, const int32_t *slot_host,
                                   int pool_slots, float *state_pool, float *checkpoints,
                                   void *o, void *stream) {
    const char *what = "gdr_decode_tokens_fused";
    if (!(gate_scale >= 0.f))   // also rejects NaN
        return fail(GDR_EINVAL, "%s: gate_scale = %g; it must be >= 0", what, (double)gate_scale);
    return decode_tokens_impl(what, dt, gk, B, n_tok, H, Dk, Dv, scale, q, k, v, gate_logit,
                              beta_logit, true, gate_scale, slot, slot_host, pool_slots,
                              state_pool, checkpoints, o, stream);
}


}  // extern "C"

namespace {

// Backward workspace for N sequences, `tokens` tokens and `chunks` chunk
// slots (fixed length: N ceil(T / 64); packed: the bound tokens / 64 + N):
// the chunk-entering states and the chunk state gradients ([chunks, H, Dv,
// Dk] fp32 each), the forward's own workspace (its schedule and chunk_base
// are reused) and the adjoint chain's per-chunk records.  The forward runs
// without storing its outputs.
struct BwdWs {
    size_t states, dstates, fwd, recs, total;
};
BwdWs bwd_layout(int gk, int N, long long tokens, long long chunks, int H, int Dk, int Dv) {
    BwdWs w{};
    if (N <= 0 || tokens <= 0 || chunks <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return w;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t st = (size_t)chunks * H * Dv * Dk * sizeof(float);
    w.states = 0;
    w.dstates = st;
    w.fwd = 2 * st;
    w.recs = w.fwd + r256(ws_layout(gk == GDR_GATE_SCALAR, true, N, tokens, H).total);
    w.total = w.recs + (size_t)chunks * H * gdr::backward_record_bytes(Dk);
    return w;
}
long long fixed_chunks(int B, int T) { return (long long)B * ((T + 63) / 64); }
long long packed_chunks(int N, long long tokens) { return tokens / 64 + N; }

}  // namespace

extern "C" {

size_t gdr_backward_workspace_bytes(enum gdr_gate gk, int B, int T, int H, int Dk, int Dv) {
    return bwd_layout(gk, B, (long long)B * T, fixed_chunks(B, T), H, Dk, Dv).total;
}

size_t gdr_backward_varlen_workspace_bytes(enum gdr_gate gk, int N, long long tokens, int H,
                                           int Dk, int Dv) {
    return bwd_layout(gk, N, tokens, packed_chunks(N, tokens), H, Dk, Dv).total;
}

gdr_status gdr_backward_chunked(enum gdr_dtype dt, enum gdr_gate gk, int B, int T, int H,
                                int Dk, int Dv, int chunk, float scale, const void *q,
                                const void *k, const void *v, const float *g,
                                const float *beta, const float *h0, const void *d_o,
                                const float *dht, float *dq, float *dk, float *dv, float *dg,
                                float *dbeta, float *dh0, void *workspace, size_t ws_bytes,
                                void *stream) {
    const char *what = "gdr_backward_chunked";
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (dt != GDR_BF16)
        return fail(GDR_EUNSUPPORTED, "%s: only bf16 inputs have a backward", what);
    if (chunk != 64) return fail(GDR_EUNSUPPORTED, "%s: chunk = %d; only 64 is supported", what, chunk);
    if (B < 0 || T < 0 || H <= 0)
        return fail(GDR_EINVAL, "%s: bad sizes B=%d T=%d H=%d", what, B, T, H);
    if ((long long)B * T * H * Dk >= (1LL << 40))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    if ((long long)B * H * 8 >= (1LL << 31) || (long long)B * ((T + 63) / 64) * H >= (1LL << 31))
        return fail(GDR_EUNSUPPORTED, "%s: grid too large", what);
    if ((long long)B * T > 0) {
        REQUIRE_PTR(q, "q");
        REQUIRE_PTR(k, "k");
        REQUIRE_PTR(v, "v");
        REQUIRE_PTR(g, "g");
        if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
        REQUIRE_PTR(d_o, "do");
        REQUIRE_PTR(dq, "dq");
        REQUIRE_PTR(dk, "dk");
        REQUIRE_PTR(dv, "dv");
        if (!dg) return fail(GDR_EINVAL, "%s: dg is NULL", what);
        if (!dbeta) return fail(GDR_EINVAL, "%s: dbeta is NULL", what);
    }
    REQUIRE_ALIGNED_OR_NULL(h0, "h0");
    REQUIRE_ALIGNED_OR_NULL(dht, "dht");
    REQUIRE_ALIGNED_OR_NULL(dh0, "dh0");
    const BwdWs W = bwd_layout(gk, B, (long long)B * T, fixed_chunks(B, T), H, Dk, Dv);
    const size_t need = W.total;
    st = check_workspace(what, workspace, ws_bytes, need);
    if (st != GDR_OK) return st;
    if (B == 0) return GDR_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        // no tokens: dS_0 = dS_T
        if (!dh0) return GDR_OK;
        return finish(gdr::launch_copy_or_zero(dh0, dht, (size_t)B * H * Dv * Dk, s), s, what);
    }
    char *ws = static_cast<char *>(workspace);
    // 1. the forward, keeping the state that enters every chunk
    const bool tiles = gk == GDR_GATE_SCALAR;
    const WsLayout FL = ws_layout(tiles, true, B, (long long)B * T, H);
    gdr::PrefillArgs f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.h0 = h0;
    f.o = nullptr; f.ht = nullptr;
    f.cu_seqlens = nullptr; f.order = nullptr; f.chunk_base = nullptr;
    f.tiles = tiles ? ws + W.fwd + FL.tiles : nullptr;
    f.unit_wide = reinterpret_cast<int32_t *>(ws + W.fwd + FL.units);
    f.max_chunks = tiles ? (long long)B * ((T + 63) / 64) : 0;
    f.N = B; f.T = T; f.H = H; f.scale = scale; f.channel_gate = gk == GDR_GATE_CHANNEL;
    f.states = reinterpret_cast<float *>(ws + W.states);
    hipError_t e = gdr::launch_prefill_chunked(Dk, f, s);
    if (e != hipSuccess) return finish(e, s, what);
    // 2, 3. the adjoint pass and the chunk gradients
    gdr::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dout = d_o; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.states = reinterpret_cast<float *>(ws + W.states);
    a.dstates = reinterpret_cast<float *>(ws + W.dstates);
    a.recs = ws + W.recs;
    a.unit_wide = f.unit_wide;
    a.cu_seqlens = nullptr; a.chunk_base = nullptr; a.chunks = fixed_chunks(B, T);
    a.B = B; a.T = T; a.H = H; a.nc = (T + 63) / 64; a.scale = scale;
    a.channel_gate = gk == GDR_GATE_CHANNEL;
    return finish(gdr::launch_backward(Dk, a, s), s, what);
}

gdr_status gdr_backward_chunked_varlen(enum gdr_dtype dt, enum gdr_gate gk, int N, int T_total,
                                       int H, int Dk, int Dv, int chunk, float scale,
                                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, const float *h0,
                                       const void *d_o, const float *dht, float *dq, float *dk,
                                       float *dv, float *dg, float *dbeta, float *dh0,
                                       void *workspace, size_t ws_bytes, void *stream) {
    const char *what = "gdr_backward_chunked_varlen";
    gdr_status st = check_common(dt, gk, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (dt != GDR_BF16)
        return fail(GDR_EUNSUPPORTED, "%s: only bf16 inputs have a backward", what);
    if (chunk != 64) return fail(GDR_EUNSUPPORTED, "%s: chunk = %d; only 64 is supported", what, chunk);
    if (N < 0 || T_total < 0 || H <= 0)
        return fail(GDR_EINVAL, "%s: bad sizes N=%d T_total=%d H=%d", what, N, T_total, H);
    if ((long long)T_total * H * Dk >= (1LL << 40))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    const long long chunks = packed_chunks(N, T_total);
    if ((long long)N * H * 8 >= (1LL << 31) || chunks * H >= (1LL << 31))
        return fail(GDR_EUNSUPPORTED, "%s: grid too large", what);
    if (N == 0) return GDR_OK;
    if (!cu_seqlens) return fail(GDR_EINVAL, "%s: cu_seqlens is NULL", what);
    if (cu_seqlens_host) {
        if (cu_seqlens_host[0] != 0)
            return fail(GDR_EINVAL, "%s: cu_seqlens[0] = %d, expected 0", what, cu_seqlens_host[0]);
        for (int i = 0; i < N; ++i)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
                return fail(GDR_EINVAL, "%s: cu_seqlens decreases at %d", what, i);
        if (cu_seqlens_host[N] != T_total)
            return fail(GDR_EINVAL, "%s: cu_seqlens[N] = %d but T_total = %d", what,
                        cu_seqlens_host[N], T_total);
    }
    if (T_total > 0) {
        REQUIRE_PTR(q, "q");
        REQUIRE_PTR(k, "k");
        REQUIRE_PTR(v, "v");
        REQUIRE_PTR(g, "g");
        if (!beta) return fail(GDR_EINVAL, "%s: beta is NULL", what);
        REQUIRE_PTR(d_o, "do");
        REQUIRE_PTR(dq, "dq");
        REQUIRE_PTR(dk, "dk");
        REQUIRE_PTR(dv, "dv");
        if (!dg) return fail(GDR_EINVAL, "%s: dg is NULL", what);
        if (!dbeta) return fail(GDR_EINVAL, "%s: dbeta is NULL", what);
    }
    REQUIRE_ALIGNED_OR_NULL(h0, "h0");
    REQUIRE_ALIGNED_OR_NULL(dht, "dht");
    REQUIRE_ALIGNED_OR_NULL(dh0, "dh0");
    const BwdWs W = bwd_layout(gk, N, T_total, chunks, H, Dk, Dv);
    st = check_workspace(what, workspace, ws_bytes, W.total);
    if (st != GDR_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T_total == 0) {
        // no tokens in any sequence: dS_0 = dS_T
        if (!dh0) return GDR_OK;
        return finish(gdr::launch_copy_or_zero(dh0, dht, (size_t)N * H * Dv * Dk, s), s, what);
    }
    char *ws = static_cast<char *>(workspace);
    const bool tiles = gk == GDR_GATE_SCALAR;
    const WsLayout FL = ws_layout(tiles, true, N, T_total, H);
    int32_t *order = reinterpret_cast<int32_t *>(ws + W.fwd + FL.order);
    int32_t *cbase = reinterpret_cast<int32_t *>(ws + W.fwd + FL.chunk_base);
    // 1. the forward (longest sequences first), keeping the state that
    //    enters every chunk at its global chunk index
    hipError_t e = gdr::launch_varlen_schedule(cu_seqlens, N, order, s);
    if (e == hipSuccess) e = gdr::launch_chunk_base(cu_seqlens, N, cbase, s);
    if (e != hipSuccess) return finish(e, s, what);
    gdr::PrefillArgs f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.h0 = h0;
    f.o = nullptr; f.ht = nullptr;
    f.cu_seqlens = cu_seqlens; f.order = order; f.chunk_base = cbase;
    f.tiles = tiles ? ws + W.fwd + FL.tiles : nullptr;
    f.unit_wide = reinterpret_cast<int32_t *>(ws + W.fwd + FL.units);
    f.max_chunks = FL.max_chunks;
    f.N = N; f.T = 0; f.H = H; f.scale = scale; f.channel_gate = gk == GDR_GATE_CHANNEL;
    f.states = reinterpret_cast<float *>(ws + W.states);
    e = gdr::launch_prefill_chunked(Dk, f, s);
    if (e != hipSuccess) return finish(e, s, what);
    // 2, 3. the adjoint pass and the chunk gradients
    gdr::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dout = d_o; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.states = reinterpret_cast<float *>(ws + W.states);
    a.dstates = reinterpret_cast<float *>(ws + W.dstates);
    a.recs = ws + W.recs;
    a.unit_wide = f.unit_wide;
    a.cu_seqlens = cu_seqlens; a.chunk_base = cbase; a.chunks = chunks;
    a.B = N; a.T = 0; a.H = H; a.nc = 0; a.scale = scale;
    a.channel_gate = gk == GDR_GATE_CHANNEL;
    return finish(gdr::launch_backward(Dk, a, s), s, what);
}

gdr_status gdr_decode_commit(int B, int n_tok, int H, int Dk, int Dv, const int32_t *slot,
                             int pool_slots, const int32_t *accepted, const float *checkpoints,
                             float *state_pool, void *stream) {
    const char *what = "gdr_decode_commit";
    gdr_status st = check_common(GDR_F32, GDR_GATE_SCALAR, Dk, Dv, what);
    if (st != GDR_OK) return st;
    if (B < 0 || n_tok < 0 || H <= 0 || pool_slots < 0)
        return fail(GDR_EINVAL, "%s: bad sizes B=%d n_tok=%d H=%d pool_slots=%d", what, B,
                    n_tok, H, pool_slots);
    if ((long long)B * H >= (1LL << 27) || (long long)pool_slots * H >= (1LL << 31))
        return fail(GDR_EUNSUPPORTED, "%s: problem too large", what);
    if (!slot && pool_slots < B)
        return fail(GDR_EINVAL, "%s: without a slot map the pool needs B = %d slots, has %d",
                    what, B, pool_slots);
    if (B == 0 || n_tok == 0) return GDR_OK;
    if (!accepted) return fail(GDR_EINVAL, "%s: accepted is NULL", what);
    REQUIRE_PTR(checkpoints, "checkpoints");
    REQUIRE_PTR(state_pool, "state_pool");
    gdr::TokensArgs a{};
    a.slot = slot; a.pool = pool_slots; a.state = state_pool;
    a.ckpt = const_cast<float *>(checkpoints);
    a.B = B; a.n = n_tok; a.H = H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdr::launch_decode_commit(Dk, a, accepted, s), s, what);
}

}  // extern "C"
