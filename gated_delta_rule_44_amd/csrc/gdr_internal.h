// gdr_internal.h -- shared declarations of libgdr's HIP kernels (gfx950).
// Internal to the library: the public interface is include/gdr.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxLayers = 1024;

// Element loads/stores for the two input dtypes (bf16 <-> fp32 conversions
// are exact one way and round-to-nearest-even the other).
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static inline float load(const float *p) { return *p; }
    __device__ static inline void store(float *p, float x) { *p = x; }
    // four consecutive values starting at p (16-byte aligned for fp32)
    __device__ static inline f32x4 load4(const float *p) {
        return *reinterpret_cast<const f32x4 *>(p);
    }
};
template <> struct Elem<bf16> {
    __device__ static inline float load(const bf16 *p) { return (float)*p; }
    __device__ static inline void store(bf16 *p, float x) { *p = (bf16)x; }
    __device__ static inline f32x4 load4(const bf16 *p) {
        bf16x4 h = *reinterpret_cast<const bf16x4 *>(p);
        return f32x4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
    }
};

// Fused input preprocessing: the kernels can take raw projections and form
// the recurrence inputs themselves, per token and head,
//     q <- q / sqrt(|q|^2 + kNormEps),  k likewise,
//     beta = 1 / (1 + e^{-x_beta}),     g = -c ln(1 + e^{x_g}),
// with the logits stored in the dtype of q.
constexpr float kNormEps = 1e-6f;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// Floor on the gate log in the chunked forms.  The chunked forms take
// differences of in-chunk prefix sums of g, which need finite terms: a gate
// a = 0 (g = -inf) would make them -inf - (-inf).  Raising every g below
// the floor to it replaces a < e^{-30} (about 9.4e-14) by e^{-30}, which
// changes each state by at most that fraction of its previous value -- far
// below fp32 rounding -- and keeps the prefix sums of a 64-token chunk above
// -1920, where fp32 differences of them are good to about 1e-4.
constexpr float kGateFloor = -30.f;

__device__ inline float logistic(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2eF));
}
// -c softplus(x) = -c (max(x, 0) + ln(1 + e^{-|x|})); v_log_f32 is log2
__device__ inline float neg_softplus(float x, float c) {
    const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2eF);
    return -c * (__builtin_fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2F);
}
__device__ inline float inv_norm(float sum_sq) {
    return __builtin_amdgcn_rsqf(sum_sq + kNormEps);
}

// One recurrent layer slot for the decode kernel: layer index and gate kind.
struct DecodeLayers {
    int n;                        // number of layers to step
    uint16_t code[kMaxLayers];    // (layer << 1) | channel_gate
};

struct DecodeArgs {
    const void *q, *k, *v;        // [L, B, H, D] dt
    const float *g;               // gate logs, see g_bh / g_layer
    const float *beta;            // [L, B, H]
    float *state;                 // [L, B, H, D, D]
    void *o;                      // [L, B, H, D] dt
    int B, H;
    float scale;
    long long g_bh;               // stride of g between (b,h) pairs (D or 1)
    long long g_layer;            // stride of g between layers
};

hipError_t launch_decode(bool bf16_io, int D, const DecodeArgs &a,
                         const DecodeLayers &layers, hipStream_t s);

// Several tokens per sequence in one launch, state in a slot-indexed pool.
struct TokensArgs {
    const void *q, *k, *v;        // [B, n, H, D] dt
    const float *g;               // [B, n, H] or [B, n, H, D]
    const float *beta;            // [B, n, H]
    const int32_t *slot;          // [B] pool slot of each sequence, or nullptr (slot b)
    long long pool;               // slots in state
    float *state;                 // [pool, H, D, D]
    float *ckpt;                  // [B, n, H, D, D] state after each token, or nullptr
    void *o;                      // [B, n, H, D] dt
    int B, n, H;
    float scale;
    int channel_gate;
    // raw projections (fused preprocessing): logits in dt, laid out as g
    // and beta; q and k are normalised in the kernel
    const void *xg, *xb;
    float gate_scale;
    // prefill form: sequence b starts from init[b] ([B, H, D, D]) instead of
    // its pool slot, or from zeros when init_zero is set; the final state
    // still goes to the slot
    const float *init;
    int init_zero;
};

hipError_t launch_decode_tokens(bool bf16_io, int D, const TokensArgs &a, hipStream_t s,
                                bool raw = false);
// state[slot[b], h] <- ckpt[b, accepted[b] - 1, h] where 1 <= accepted[b] <= n
hipError_t launch_decode_commit(int D, const TokensArgs &a, const int32_t *accepted,
                                hipStream_t s);

// Fixed-length (cu_seqlens == nullptr, T = seq_len) or packed batches.
struct PrefillArgs {
    const void *q, *k, *v;        // [tokens, H, D] dt
    const float *g;               // [tokens, H] or [tokens, H, D]
    const float *beta;            // [tokens, H]
    const float *h0;              // [N, H, D, D] or nullptr
    void *o;                      // [tokens, H, D] dt; bf16 chunked forms: nullptr = not stored
    float *ht;                    // [N, H, D, D] or nullptr
    const int32_t *cu_seqlens;    // [N+1] or nullptr (fixed length)
    const int32_t *order;         // schedule [N] or nullptr (identity)
    int32_t *chunk_base;          // varlen: first chunk of each sequence [N+1] (written)
    void *tiles;                  // scalar gate: one kTileBytes record per (chunk, head)
    // one int32 per (sequence, head) [N, H]: 1 where some chunk decays by
    // more than e^80 in some channel.  Channel gate, bf16: written by the
    // plain pass and read by the reference pass, which redoes those pairs;
    // scalar gate: written by the recurrence kernel when set (the backward
    // reads it), otherwise nullptr
    int32_t *unit_wide;
    long long max_chunks;         // chunk records per head in tiles
    int N, T, H;                  // T used only when cu_seqlens == nullptr
    float scale;
    int channel_gate;
    // pool form: h0 == ht == a [pool, H, D, D] state pool, sequence n starts
    // from slot h0_slot[n] and ends in slot ht_slot[n]; nullptr = slot n
    const int32_t *h0_slot, *ht_slot;
    long long pool;
    // raw projections (fused preprocessing) when xg != nullptr: gate and
    // beta logits in the dtype of q, laid out as g and beta; q and k are
    // normalised in the kernels
    const void *xg, *xb;
    float gate_scale;
    // bf16 path only: when set, the state entering every chunk of every
    // (sequence, head), [chunks, H, D, D] fp32 at global chunk
    // chunk_base[n] + c (fixed length: n ceil(T / 64) + c; packed batches
    // need chunk_base filled) -- for the backward
    float *states;
};

// Initial state of sequence n, head h (nullptr: start from zeros) and where
// its final state goes (nullptr: not stored).  A pool slot outside
// [0, pool) selects zeros / no store.
template <int D>
__device__ inline const float *seq_h0(const PrefillArgs &a, int n, int h) {
    long long s = n;
    if (a.h0_slot) {
        s = a.h0_slot[n];
        if (s < 0 || s >= a.pool) return nullptr;
    }
    return a.h0 ? a.h0 + ((size_t)s * a.H + h) * D * D : nullptr;
}
template <int D>
__device__ inline float *seq_ht(const PrefillArgs &a, int n, int h) {
    long long s = n;
    if (a.ht_slot) {
        s = a.ht_slot[n];
        if (s < 0 || s >= a.pool) return nullptr;
    }
    return a.ht ? a.ht + ((size_t)s * a.H + h) * D * D : nullptr;
}

// Per (chunk, head) record of the scalar-gate chunked prefill's workspace:
// T as MFMA operands of its 16x16 blocks (bf16, 5 KiB), then three fp32 rows
// over the chunk's 64 tokens: the gate prefix sums b_r log2(e) and the
// decay factors e^{b_C - b_r} and e^{b_r}.
constexpr size_t kTileBytes = 5 * 1024 + 3 * 64 * 4;
// With fused preprocessing the record carries the key norms as one more
// row and folds them into the last two (6 KiB).
constexpr size_t kTileBytesRaw = kTileBytes + 64 * 4;

// Backward of the chunked prefill (bf16 q/k/v/do), a fixed-length batch
// (cu_seqlens == nullptr: B sequences of T tokens, nc = ceil(T / 64) chunks
// each) or a packed one (B sequences, cu_seqlens [B+1], chunk_base [B+1]
// their first global chunks).  Per-chunk workspace is indexed
// [global chunk][head]: sequence n's chunk c is global chunk
// chunk_base[n] + c (fixed length: n nc + c).
struct BwdArgs {
    const void *q, *k, *v;        // [tokens, H, D] bf16
    const float *g, *beta;        // [tokens, H(, D)], [tokens, H]
    const float *h0;              // [B, H, D, D] or nullptr
    const void *dout;             // [tokens, H, D] bf16: gradient of o
    const float *dht;             // [B, H, D, D] or nullptr: gradient of the final state
    float *dq, *dk, *dv;          // [tokens, H, D]
    float *dg, *dbeta;            // like g, beta
    float *dh0;                   // [B, H, D, D] or nullptr
    float *states, *dstates;      // workspace: [chunks, H, D, D] each
    void *recs;                   // workspace: one record per (global chunk, head)
    const int32_t *cu_seqlens;    // [B+1] or nullptr (fixed length)
    const int32_t *chunk_base;    // [B+1] (packed batches)
    long long chunks;             // global chunks the grid covers (an upper bound when packed)
    // [B, H]: pairs the forward marked (a chunk decays by more than e^80 in
    // some channel); their gradients are recomputed by the token-level
    // adjoint.  nullptr: none marked.
    const int32_t *unit_wide;
    int B, T, H, nc;              // T, nc: fixed length only
    float scale;
    int channel_gate;
};
// chunk_base[n] = sum over m < n of ceil(len_m / 64), n = 0..N
hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *chunk_base,
                             hipStream_t s);
hipError_t launch_backward(int D, const BwdArgs &a, hipStream_t s);
hipError_t launch_copy_or_zero(float *dst, const float *src, size_t n, hipStream_t s);
size_t backward_record_bytes(int D);

hipError_t launch_prefill_recurrent(bool bf16_io, int D, const PrefillArgs &a,
                                    hipStream_t s);
hipError_t launch_prefill_chunked(int D, const PrefillArgs &a, hipStream_t s);
// scalar gate: the state chain on dedicated waves (chunked_chain.hip)
hipError_t launch_prefill_chain(int D, const PrefillArgs &a, hipStream_t s);
hipError_t launch_varlen_schedule(const int32_t *cu_seqlens, int N,
                                  int32_t *order, hipStream_t s);

}  // namespace gdr
