// recurrent.hip -- fused single-token state update (decode) and the
// token-by-token prefill that repeats it, for gfx950.
//
// Per (sequence, head) and token, with the gate given as g = ln a:
//     S' = S Diag(a);   u = beta (v - S' k);   S <- S' + u k^T;
//     o  = scale * S q = scale * (S' q + u (k.q))
// which is the gated delta rule S_t = S_{t-1} Diag(a_t)(I - beta k k^T)
// + beta v k^T, o_t = S_t q_t, multiplied out (Kimi Delta Attention: a per
// key channel; Gated DeltaNet: one scalar a per head -- "Super Apriel: One
// Checkpoint, Many Speeds", gist.science summary, section 2a).
//
// Layout.  A state row is D floats = D/4 lanes of float4, so a 64-lane wave
// covers 64/(D/4) rows per load and every load instruction of a 256-thread
// workgroup reads one contiguous block of rows: the state streams from HBM
// with dwordx4 accesses, once in and once out.  The decode spreads one state
// over several workgroups (rows are independent); the recurrent prefill keeps
// a whole state in one workgroup, thread (wave w, lane l) holding rows
//     row(m) = m * RPI + w * RPW + l / LPR,   m < M
// at columns 4 * (l % LPR) .. +3, and reduces its 2M row dot products (S'k
// and S'q) by a recursive-halving exchange across the LPR lanes of a row,
// which leaves one finished dot product per lane.
#include "gdr_internal.h"
#include "device_util.h"

#ifndef GDR_DECODE_PASSES
#define GDR_DECODE_PASSES 2   // 16 rows (8 KiB of state) per workgroup at D = 128
#endif

namespace gdr {
namespace {

template <int D> struct Geom {
    static constexpr int LPR = D / 4;          // lanes per state row
    static constexpr int RPW = 64 / LPR;       // rows per wave per load
    static constexpr int NW = 4;               // waves per workgroup
    static constexpr int RPI = RPW * NW;       // rows per workgroup load
    static constexpr int M = D / RPI;          // rows held per thread
    static constexpr int NV = 2 * M;           // dot products per thread
    static constexpr int LOG_LPR = D == 128 ? 5 : 4;
    static constexpr int LOG_NV = D == 128 ? 5 : 3;
    static constexpr int SHIFT = LOG_LPR - LOG_NV;   // lanes sharing a result
    static_assert(LPR >= NV, "reduce-scatter needs one lane per result");
};

__device__ inline float dot4(f32x4 a, f32x4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// One token's inputs as this thread needs them: k and q at its four columns,
// the gate logs there (a scalar gate: its one value four times), v at the
// row whose dot products the thread finishes, and beta.  RAW (fused
// preprocessing): the gate and beta logits instead, and q and k not yet
// normalised.
struct StepIn {
    f32x4 kv, qv, lg;
    float vrow, beta;
};

// Row of the result a thread finishes in head_step (see there)
template <int D>
__device__ inline int result_row(int lane, int w) {
    using G = Geom<D>;
    const int idx = (lane % G::LPR) >> G::SHIFT;
    return (idx % G::M) * G::RPI + w * G::RPW + lane / G::LPR;
}

// qp, kp, vp point at the head's D-vector for the token, gp at its gate logs
// (D values for a channel gate, one for a scalar gate; fp32, or type T
// logits with RAW), bp at its beta (RAW: a type T logit)
template <typename T, int D, bool RAW, bool CH>
__device__ inline StepIn step_load(const T *qp, const T *kp, const T *vp, const void *gp,
                                   const void *bp, int lane, int w) {
    using G = Geom<D>;
    const int c0 = (lane % G::LPR) * 4;
    StepIn x;
    x.kv = Elem<T>::load4(kp + c0);
    x.qv = Elem<T>::load4(qp + c0);
    // a scalar gate (CH false) is loaded into lg.x alone and broadcast
    // where it is used, so that no copy waits for the load
    if (RAW) {
        const T *xg = static_cast<const T *>(gp);
        if constexpr (CH) x.lg = Elem<T>::load4(xg + c0);
        else              x.lg.x = Elem<T>::load(xg);
        x.beta = Elem<T>::load(static_cast<const T *>(bp));
    } else {
        const float *g = static_cast<const float *>(gp);
        if constexpr (CH) x.lg = *reinterpret_cast<const f32x4 *>(g + c0);
        else              x.lg.x = g[0];
        x.beta = *static_cast<const float *>(bp);
    }
    x.vrow = Elem<T>::load(vp + result_row<D>(lane, w));
    return x;
}

// Cross-lane steps of head_step when a state row is one 16-lane DPP row
// (D = 64): VALU data-parallel moves instead of LDS permutes.  Recursive
// halving needs, at the level of lane bit b, a partner with bit b flipped
// and the higher bits kept (it holds the same part of the list); row_mirror
// (lane i <-> 15 - i), row_half_mirror (i <-> i ^ 7 within each 8) and the
// quad permutes xor 2, xor 1 are such partners for b = 8, 4, 2, 1, and the
// lane keeps the part its own bit selects, so every lane ends with the sum
// over all 16 lanes of the result its bits name.
template <int MASK, int CTRL, int NV>
__device__ inline void halving_step(float (&val)[NV], int &n, int lane) {
    if (n > 1) {
        const int half = n / 2;
        const bool upper = (lane & MASK) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float keep = upper ? val[half + i] : val[i];
            const float give = upper ? val[i] : val[half + i];
            val[i] = keep + dpp_f<CTRL>(give);
        }
        n = half;
    } else {
        val[0] += dpp_f<CTRL>(val[0]);
    }
}
// u of lane 2 m of each 16-lane row (row_newbcast), for the M rows m
template <int M, int SHIFT, int m = 0>
__device__ inline void bcast_rows(float u, float (&um)[M]) {
    if constexpr (m < M) {
        um[m] = dpp_f<0x150 + (m << SHIFT)>(u);
        bcast_rows<M, SHIFT, m + 1>(u, um);
    }
}

// One token's update of the state slice S held by this thread, from the
// token's inputs; the output is written to op.
template <typename T, int D, bool RAW, bool CH>
__device__ inline void head_step(f32x4 (&S)[Geom<D>::M], StepIn in, float scale,
                                 float gate_scale, T *op, int lane, int w) {
    using G = Geom<D>;
    constexpr bool kDpp = G::LPR == 16;          // a state row is one DPP row
    const int sub = lane / G::LPR;
    f32x4 kv = in.kv, qv = in.qv, lg = in.lg;
    float beta = in.beta;
    if (RAW) {
        if constexpr (CH)
            lg = f32x4{neg_softplus(lg.x, gate_scale), neg_softplus(lg.y, gate_scale),
                       neg_softplus(lg.z, gate_scale), neg_softplus(lg.w, gate_scale)};
        else
            lg.x = neg_softplus(lg.x, gate_scale);
        beta = logistic(beta);
        float sk = dot4(kv, kv), sq = dot4(qv, qv);
        if constexpr (kDpp) {
            sk = sum_group<16>(sk);
            sq = sum_group<16>(sq);
        } else {
#pragma unroll
            for (int mask = G::LPR / 2; mask >= 1; mask >>= 1) {
                sk += __shfl_xor(sk, mask);
                sq += __shfl_xor(sq, mask);
            }
        }
        kv = kv * inv_norm(sk);
        qv = qv * inv_norm(sq);
    }
    if constexpr (!CH) lg = f32x4{lg.x, lg.x, lg.x, lg.x};
    constexpr float kLog2e = 1.4426950408889634f;
    const f32x4 a = f32x4{__builtin_amdgcn_exp2f(lg.x * kLog2e),
                          __builtin_amdgcn_exp2f(lg.y * kLog2e),
                          __builtin_amdgcn_exp2f(lg.z * kLog2e),
                          __builtin_amdgcn_exp2f(lg.w * kLog2e)};
    const f32x4 ak = a * kv;
    const f32x4 aq = a * qv;

    // k.q over the full row: all-reduce across the LPR lanes of the row
    float kq = dot4(kv, qv);
    if constexpr (kDpp) {
        kq = sum_group<16>(kq);
    } else {
#pragma unroll
        for (int mask = G::LPR / 2; mask >= 1; mask >>= 1)
            kq += __shfl_xor(kq, mask);
    }

    // partial (S'k)_row and (S'q)_row over this thread's 4 columns
    float val[G::NV];
#pragma unroll
    for (int m = 0; m < G::M; ++m) {
        val[m] = dot4(S[m], ak);
        val[G::M + m] = dot4(S[m], aq);
    }
    // recursive halving: after step with mask b the lane keeps the half of
    // the list selected by its lane bit b, summed with the partner's copy
    int n = G::NV;
    if constexpr (kDpp) {
        halving_step<8, 0x140>(val, n, lane);   // row_mirror
        halving_step<4, 0x141>(val, n, lane);   // row_half_mirror
        halving_step<2, 0x4E>(val, n, lane);    // quad_perm [2,3,0,1]
        halving_step<1, 0xB1>(val, n, lane);    // quad_perm [1,0,3,2]
    } else {
#pragma unroll
        for (int mask = G::LPR / 2; mask >= 1; mask >>= 1) {
            if (n > 1) {
                const int half = n / 2;
                const bool upper = (lane & mask) != 0;
#pragma unroll
                for (int i = 0; i < half; ++i) {
                    const float keep = upper ? val[half + i] : val[i];
                    const float give = upper ? val[i] : val[half + i];
                    val[i] = keep + __shfl_xor(give, mask);
                }
                n = half;
            } else {
                val[0] += __shfl_xor(val[0], mask);
            }
        }
    }
    // this lane now holds result index idx: which = idx / M, row slot idx % M
    // (row result_row(lane, w))
    const int idx = (lane % G::LPR) >> G::SHIFT;
    const bool is_q = idx >= G::M;
    const int row = result_row<D>(lane, w);

    const float u = beta * (in.vrow - val[0]);           // valid where !is_q
    float u_pair;                                        // for is_q lanes
    if constexpr (kDpp) {
        static_assert((G::M << G::SHIFT) == 8, "partner of the k result: lane ^ 8");
        u_pair = dpp_f<0x128>(u);                        // row_ror:8 = lane ^ 8 in a row
    } else {
        u_pair = __shfl_xor(u, G::M << G::SHIFT);
    }
    if (is_q && (lane & ((1 << G::SHIFT) - 1)) == 0)
        Elem<T>::store(op + row, scale * (val[0] + u_pair * kq));

    // rank-1 update: every lane needs u for each of its M rows
    float um[G::M];
    if constexpr (kDpp) {
        bcast_rows<G::M, G::SHIFT>(u, um);
    } else {
#pragma unroll
        for (int m = 0; m < G::M; ++m) um[m] = __shfl(u, sub * G::LPR + (m << G::SHIFT));
    }
#pragma unroll
    for (int m = 0; m < G::M; ++m) S[m] = S[m] * a + um[m] * kv;
}

// Consecutive workgroups go to the eight XCDs in turn, each with its own L2.
// The NRB workgroups of one head share its q, k and gate vectors, so they
// are numbered to run on one XCD, two heads after another: each XCD then
// streams 2 * D * D * 4 contiguous bytes of state per run, and all but the
// first workgroup of a head find its vectors in L2 (measured on the
// 48-layer decode: 4.45 ms with heads spread over XCDs, 4.18 ms with one
// head per run, 4.01 ms with two, 4.11 ms with four).  Heads beyond the
// last multiple of 16 keep the plain order.
template <int NRB>
__device__ inline void xcd_head_block(int i, long long heads, int &head, int &rb) {
    constexpr int G = 2;                       // heads per run on one XCD
    const long long full = (heads / (8 * G)) * 8 * G * NRB;
    if (i < full) {
        const int x = i & 7, j = i >> 3;
        const int run = j / (NRB * G), r = j % (NRB * G);
        head = (run * 8 + x) * G + r / NRB;
        rb = r % NRB;
    } else {
        head = i / NRB;
        rb = i % NRB;
    }
}

template <int D>
__device__ inline const float *state_row(const float *st, int m, int lane, int w) {
    using G = Geom<D>;
    const int row = m * G::RPI + w * G::RPW + lane / G::LPR;
    return st + (size_t)row * D + (lane % G::LPR) * 4;
}

// ---------------------------------------------------------------------------
// Decode, row-split: the rows of one state are independent (each row's dot
// products need only that row and the head's shared q, k and gate), so a
// head is spread over D / ROWS workgroups of ROWS rows each.  Small
// per-workgroup footprints keep many independent read-then-write streams in
// flight, which measures markedly faster than one 64 KiB state per
// workgroup.  Thread (wave w, lane l) holds row
//     rowblock * ROWS + p * RPP + w * RPW + l / LPR,  p < PASSES,
// columns 4 * (l % LPR) .. +3.
template <typename T, int D, int PASSES>
__global__ __launch_bounds__(256) void decode_rows_kernel(DecodeArgs a, DecodeLayers L) {
    using G = Geom<D>;
    constexpr int RPP = G::RPI;              // rows per pass of the workgroup
    constexpr int ROWS = RPP * PASSES;
    constexpr int NRB = D / ROWS;            // workgroups per head
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int bh_count = a.B * a.H;
    int rb, slot_lin;
    xcd_head_block<NRB>(blockIdx.x, (long long)L.n * bh_count, slot_lin, rb);
    const int rec = slot_lin / bh_count;
    const int bh = slot_lin - rec * bh_count;
    const int code = L.code[rec];
    const int layer = code >> 1;
    const bool channel = (code & 1) != 0;
    const size_t slot = (size_t)layer * bh_count + bh;
    const int c0 = (lane % G::LPR) * 4;
    const int sub = lane / G::LPR;

    float *st = a.state + slot * D * D;
    f32x4 S[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = rb * ROWS + p * RPP + w * G::RPW + sub;
        S[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(st + (size_t)row * D + c0));
    }
    const T *qp = static_cast<const T *>(a.q) + slot * D;
    const T *kp = static_cast<const T *>(a.k) + slot * D;
    const T *vp = static_cast<const T *>(a.v) + slot * D;
    T *op = static_cast<T *>(a.o) + slot * D;
    const float *gp = a.g + layer * a.g_layer + (long long)bh * a.g_bh;
    const float beta = a.beta[slot];
    const f32x4 kv = Elem<T>::load4(kp + c0);
    const f32x4 qv = Elem<T>::load4(qp + c0);
    f32x4 lg;
    if (channel) {
        lg = *reinterpret_cast<const f32x4 *>(gp + c0);
    } else {
        const float s = gp[0];
        lg = f32x4{s, s, s, s};
    }
    constexpr float kLog2e = 1.4426950408889634f;
    const f32x4 av = f32x4{__builtin_amdgcn_exp2f(lg.x * kLog2e), __builtin_amdgcn_exp2f(lg.y * kLog2e),
                           __builtin_amdgcn_exp2f(lg.z * kLog2e), __builtin_amdgcn_exp2f(lg.w * kLog2e)};
    const f32x4 ak = av * kv;
    const f32x4 aq = av * qv;
    float kq = dot4(kv, qv);
#pragma unroll
    for (int mask = G::LPR / 2; mask >= 1; mask >>= 1) kq += __shfl_xor(kq, mask);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = rb * ROWS + p * RPP + w * G::RPW + sub;
        // (S'k)_row and (S'q)_row: one halving step, then an all-reduce
        const float yk = dot4(S[p], ak);
        const float yq = dot4(S[p], aq);
        const bool upper = (lane & (G::LPR / 2)) != 0;
        float val = (upper ? yq : yk) + __shfl_xor(upper ? yk : yq, G::LPR / 2);
#pragma unroll
        for (int mask = G::LPR / 4; mask >= 1; mask >>= 1) val += __shfl_xor(val, mask);
        // lanes in the lower half of the row now hold S'k, the upper half S'q
        const float vrow = Elem<T>::load(vp + row);
        const float u_lo = beta * (vrow - val);
        const float u = __shfl_xor(u_lo, G::LPR / 2);
        const float um = upper ? u : u_lo;       // every lane: u for its row
        if (upper && (lane % (G::LPR / 2)) == 0) Elem<T>::store(op + row, a.scale * (val + um * kq));
        S[p] = S[p] * av + um * kv;
        __builtin_nontemporal_store(S[p], reinterpret_cast<f32x4 *>(st + (size_t)row * D + c0));
    }
}

// ---------------------------------------------------------------------------
// Several tokens per sequence in one launch (drafted tokens of speculative
// decoding, or a short continuation): the decode update above applied to
// tokens 0 .. n-1 in order with the state slice resident in registers, so
// the state is read from HBM once.  With a checkpoint buffer the state after
// every token is written there and the pool keeps its bytes (the caller
// installs the state after the accepted prefix with the commit kernel);
// without one the state after the last token replaces the pool's.  The
// state lives in a slot-indexed pool: sequence b uses slot slot[b], and a
// slot outside [0, pool) marks an idle sequence that is skipped.
template <int PASSES>
struct TokIn {
    f32x4 k, q, lg;
    float beta;
    float v[PASSES];
};

// RAW: the gate and beta slots hold the logits, still to be transformed.
// CH: a channel gate (four values per lane), else a scalar gate (in lg.x,
// broadcast where it is used, so that no copy waits for the load)
template <typename T, int D, int PASSES, bool RAW, bool CH>
__device__ __forceinline__ TokIn<PASSES> load_token(const TokensArgs &a, size_t bth, int c0,
                                                    const int (&row)[PASSES]) {
    TokIn<PASSES> x;
    const T *kp = static_cast<const T *>(a.k) + bth * D;
    const T *qp = static_cast<const T *>(a.q) + bth * D;
    const T *vp = static_cast<const T *>(a.v) + bth * D;
    x.k = Elem<T>::load4(kp + c0);
    x.q = Elem<T>::load4(qp + c0);
    if (RAW) {
        const T *xg = static_cast<const T *>(a.xg);
        if constexpr (CH) x.lg = Elem<T>::load4(xg + bth * D + c0);
        else              x.lg.x = Elem<T>::load(xg + bth);
        x.beta = Elem<T>::load(static_cast<const T *>(a.xb) + bth);
    } else {
        if constexpr (CH) x.lg = *reinterpret_cast<const f32x4 *>(a.g + bth * D + c0);
        else              x.lg.x = a.g[bth];
        x.beta = a.beta[bth];
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) x.v[p] = Elem<T>::load(vp + row[p]);
    return x;
}

template <typename T, int D, int PASSES, bool RAW, bool CH>
__global__ __launch_bounds__(256) void decode_tokens_kernel(TokensArgs a) {
    using G = Geom<D>;
    constexpr int RPP = G::RPI;
    constexpr int ROWS = RPP * PASSES;
    constexpr int NRB = D / ROWS;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int rb, bh;
    xcd_head_block<NRB>(blockIdx.x, (long long)a.B * a.H, bh, rb);
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    long long slot = b;
    if (a.slot) {
        slot = a.slot[b];
        if (slot < 0 || slot >= a.pool) return;
    }
    const int c0 = (lane % G::LPR) * 4;
    const int sub = lane / G::LPR;
    int row[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) row[p] = rb * ROWS + p * RPP + w * G::RPW + sub;

    float *st = a.state + ((size_t)slot * a.H + h) * D * D;
    const float *s0 = a.init ? a.init + ((size_t)b * a.H + h) * D * D : st;
    f32x4 S[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        S[p] = a.init_zero ? f32x4{0.f, 0.f, 0.f, 0.f}
                           : __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s0 + (size_t)row[p] * D + c0));

    const size_t bh0 = (size_t)b * a.n * a.H + h;        // (b, token 0, h)
    constexpr float kLog2e = 1.4426950408889634f;
    // a state row is one 16-lane DPP row at D = 64: VALU moves (row_ror:8
    // is lane ^ 8 within the row; quad permutes and row_half_mirror sum each
    // half) instead of LDS permutes
    constexpr bool kDpp = G::LPR == 16;
    auto step = [&](TokIn<PASSES> cur, int t) {
        const size_t bth = bh0 + (size_t)t * a.H;
        f32x4 lg = cur.lg;
        if (RAW) {
            // |k|^2 and |q|^2 over the LPR lanes of the row, then the
            // normalised vectors, beta and the gate logs from their logits
            float sk = dot4(cur.k, cur.k), sq = dot4(cur.q, cur.q);
            if constexpr (kDpp) {
                sk = sum_group<16>(sk);
                sq = sum_group<16>(sq);
            } else {
#pragma unroll
                for (int mask = G::LPR / 2; mask >= 1; mask >>= 1) {
                    sk += __shfl_xor(sk, mask);
                    sq += __shfl_xor(sq, mask);
                }
            }
            cur.k = cur.k * inv_norm(sk);
            cur.q = cur.q * inv_norm(sq);
            cur.beta = logistic(cur.beta);
            if constexpr (CH)
                lg = f32x4{neg_softplus(lg.x, a.gate_scale), neg_softplus(lg.y, a.gate_scale),
                           neg_softplus(lg.z, a.gate_scale), neg_softplus(lg.w, a.gate_scale)};
            else
                lg.x = neg_softplus(lg.x, a.gate_scale);
        }
        if constexpr (!CH) lg = f32x4{lg.x, lg.x, lg.x, lg.x};
        const f32x4 av = f32x4{__builtin_amdgcn_exp2f(lg.x * kLog2e), __builtin_amdgcn_exp2f(lg.y * kLog2e),
                               __builtin_amdgcn_exp2f(lg.z * kLog2e), __builtin_amdgcn_exp2f(lg.w * kLog2e)};
        const f32x4 ak = av * cur.k;
        const f32x4 aq = av * cur.q;
        float kq = dot4(cur.k, cur.q);
        if constexpr (kDpp) {
            kq = sum_group<16>(kq);
        } else {
#pragma unroll
            for (int mask = G::LPR / 2; mask >= 1; mask >>= 1) kq += __shfl_xor(kq, mask);
        }
        T *op = static_cast<T *>(a.o) + bth * D;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float yk = dot4(S[p], ak);
            const float yq = dot4(S[p], aq);
            const bool upper = (lane & (G::LPR / 2)) != 0;
            float val, u_lo, u;
            if constexpr (kDpp) {
                val = (upper ? yq : yk) + dpp_f<0x128>(upper ? yk : yq);
                val = sum_group<8>(val);
                u_lo = cur.beta * (cur.v[p] - val);
                u = dpp_f<0x128>(u_lo);
            } else {
                val = (upper ? yq : yk) + __shfl_xor(upper ? yk : yq, G::LPR / 2);
#pragma unroll
                for (int mask = G::LPR / 4; mask >= 1; mask >>= 1) val += __shfl_xor(val, mask);
                u_lo = cur.beta * (cur.v[p] - val);
                u = __shfl_xor(u_lo, G::LPR / 2);
            }
            const float um = upper ? u : u_lo;
            if (upper && (lane % (G::LPR / 2)) == 0) Elem<T>::store(op + row[p], a.scale * (val + um * kq));
            S[p] = S[p] * av + um * cur.k;
        }
        if (a.ckpt) {
            float *cp = a.ckpt + bth * D * D;
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                __builtin_nontemporal_store(S[p], reinterpret_cast<f32x4 *>(cp + (size_t)row[p] * D + c0));
        }
    };
    auto load = [&](int t) { return load_token<T, D, PASSES, RAW, CH>(a, bh0 + (size_t)t * a.H, c0, row); };
    if constexpr (PASSES == 1) {
        // the recurrent prefill's form (few registers, a short step): token
        // t + 2's inputs are loaded while token t is worked on, into three
        // register sets taken in turn -- token u lives in set u mod 3 -- so
        // that no set is copied while its loads are in flight
        constexpr int AH = 2, NS = 3;
        TokIn<PASSES> in[NS];
#pragma unroll
        for (int i = 0; i < AH; ++i)
            if (i < a.n) in[i] = load(i);
        int t = 0;
        // every load of a trip is in range here, so none is conditional
        for (; t + AH + NS <= a.n; t += NS) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                in[(i + AH) % NS] = load(t + i + AH);
                step(in[i], t + i);
            }
        }
        for (; t < a.n; t += NS) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                if (t + i < a.n) {
                    if (t + i + AH < a.n) in[(i + AH) % NS] = load(t + i + AH);
                    step(in[i], t + i);
                }
            }
        }
    } else {
        // the decode (two passes of rows): the next token's inputs in flight
        // while a token is worked on; more sets would cost waves per SIMD
        TokIn<PASSES> cur = load(0);
        for (int t = 0; t < a.n; ++t) {
            const TokIn<PASSES> nxt = t + 1 < a.n ? load(t + 1) : cur;
            step(cur, t);
            cur = nxt;
        }
    }
    if (!a.ckpt) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            __builtin_nontemporal_store(S[p], reinterpret_cast<f32x4 *>(st + (size_t)row[p] * D + c0));
    }
}

// Install the state after the accepted prefix: for 1 <= accepted[b] <= n the
// checkpoint of token accepted[b] - 1 replaces the pool slot's state; other
// counts (0: every drafted token rejected) leave the slot as it is.  One
// workgroup copies 16 KiB of one state.
template <int D>
__global__ __launch_bounds__(256) void commit_kernel(TokensArgs a, const int32_t *accepted) {
    constexpr int PIECE = 4096;                 // floats per workgroup
    constexpr int NP = D * D / PIECE;
    constexpr int V = PIECE / 4 / 256;          // float4 per thread
    int piece, bh;
    xcd_head_block<NP>(blockIdx.x, (long long)a.B * a.H, bh, piece);
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int m = accepted[b];
    if (m < 1 || m > a.n) return;
    long long slot = b;
    if (a.slot) {
        slot = a.slot[b];
        if (slot < 0 || slot >= a.pool) return;
    }
    const f32x4 *src = reinterpret_cast<const f32x4 *>(
        a.ckpt + (((size_t)b * a.n + (m - 1)) * a.H + h) * D * D + (size_t)piece * PIECE);
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.state + ((size_t)slot * a.H + h) * D * D +
                                           (size_t)piece * PIECE);
    f32x4 x[V];
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = __builtin_nontemporal_load(src + i * 256 + threadIdx.x);
#pragma unroll
    for (int i = 0; i < V; ++i) __builtin_nontemporal_store(x[i], dst + i * 256 + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Prefill in the recurrent form: one workgroup per (sequence, head) walks
// its tokens in order with the state resident in registers.
template <typename T, int D, bool RAW, bool CH>
__global__ __launch_bounds__(256) void prefill_recurrent_kernel(PrefillArgs a) {
    using G = Geom<D>;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int rank = blockIdx.x / a.H;
    const int h = blockIdx.x - rank * a.H;
    const int n = a.order ? a.order[rank] : rank;
    long long t0, t1;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        t1 = a.cu_seqlens[n + 1];
    } else {
        t0 = (long long)n * a.T;
        t1 = t0 + a.T;
    }
    const float *h0p = seq_h0<D>(a, n, h);

    f32x4 S[G::M];
#pragma unroll
    for (int m = 0; m < G::M; ++m)
        S[m] = h0p ? *reinterpret_cast<const f32x4 *>(state_row<D>(h0p, m, lane, w))
                   : f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t tok = (size_t)a.H * D;                 // q/k/v/o token stride
    const size_t gtok = CH ? tok : (size_t)a.H;
    const size_t goff = CH ? (size_t)h * D : (size_t)h;
    const T *q = static_cast<const T *>(a.q) + h * D;
    const T *k = static_cast<const T *>(a.k) + h * D;
    const T *v = static_cast<const T *>(a.v) + h * D;
    T *o = static_cast<T *>(a.o) + h * D;
    // token t's inputs, loaded P tokens ahead of their step (a ring of P
    // register sets, so that the load latency is paid once, not per token)
    auto load = [&](long long t) -> StepIn {
        if (RAW)
            return step_load<T, D, true, CH>(q + t * tok, k + t * tok, v + t * tok,
                                         static_cast<const T *>(a.xg) + t * gtok + goff,
                                         static_cast<const T *>(a.xb) + t * a.H + h,
                                         lane, w);
        return step_load<T, D, false, CH>(q + t * tok, k + t * tok, v + t * tok,
                                      a.g + t * gtok + goff, a.beta + t * a.H + h,
                                      lane, w);
    };
    constexpr int P = 4;
    StepIn in[P];
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (t0 + i < t1) in[i] = load(t0 + i);
    long long t = t0;
    // every load of the main loop is in range (t + 2P - 1 < t1), so none is
    // conditional there
    for (; t + 2 * P <= t1; t += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            head_step<T, D, RAW, CH>(S, in[i], a.scale, a.gate_scale, o + (t + i) * tok, lane, w);
            in[i] = load(t + i + P);
        }
    }
    for (; t < t1; t += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            if (t + i < t1) {
                head_step<T, D, RAW, CH>(S, in[i], a.scale, a.gate_scale, o + (t + i) * tok, lane, w);
                if (t + i + P < t1) in[i] = load(t + i + P);
            }
        }
    }
    if (float *htp = seq_ht<D>(a, n, h)) {
#pragma unroll
        for (int m = 0; m < G::M; ++m)
            *reinterpret_cast<f32x4 *>(const_cast<float *>(state_row<D>(htp, m, lane, w))) = S[m];
    }
}

}  // namespace

hipError_t launch_decode(bool bf16_io, int D, const DecodeArgs &a,
                         const DecodeLayers &layers, hipStream_t s) {
    const long long heads = (long long)layers.n * a.B * a.H;
    if (heads <= 0) return hipSuccess;
    // rows per workgroup: PASSES x (rows one workgroup-wide load covers)
    constexpr int P128 = GDR_DECODE_PASSES, P64 = GDR_DECODE_PASSES;
    const long long per_head = D == 128 ? 128 / (Geom<128>::RPI * P128) : 64 / (Geom<64>::RPI * P64);
    const long long blocks = heads * per_head;
    if (blocks >= (1LL << 31)) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(256);
    if (bf16_io) {
        if (D == 128) hipLaunchKernelGGL((decode_rows_kernel<bf16, 128, P128>), grid, block, 0, s, a, layers);
        else          hipLaunchKernelGGL((decode_rows_kernel<bf16, 64, P64>), grid, block, 0, s, a, layers);
    } else {
        if (D == 128) hipLaunchKernelGGL((decode_rows_kernel<float, 128, P128>), grid, block, 0, s, a, layers);
        else          hipLaunchKernelGGL((decode_rows_kernel<float, 64, P64>), grid, block, 0, s, a, layers);
    }
    return hipGetLastError();
}

// the token kernel for a dtype, D, gate kind and raw flag, P passes of rows
template <int P, bool RAW, bool CH>
void launch_tokens_p(bool bf16_io, int D, const TokensArgs &a, dim3 grid, hipStream_t s) {
    dim3 block(256);
    if (bf16_io) {
        if (D == 128) hipLaunchKernelGGL((decode_tokens_kernel<bf16, 128, P, RAW, CH>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((decode_tokens_kernel<bf16, 64, P, RAW, CH>), grid, block, 0, s, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((decode_tokens_kernel<float, 128, P, RAW, CH>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((decode_tokens_kernel<float, 64, P, RAW, CH>), grid, block, 0, s, a);
    }
}
template <int P>
void launch_tokens_any(bool bf16_io, int D, const TokensArgs &a, dim3 grid, hipStream_t s, bool raw) {
    if (raw) {
        if (a.channel_gate) launch_tokens_p<P, true, true>(bf16_io, D, a, grid, s);
        else                launch_tokens_p<P, true, false>(bf16_io, D, a, grid, s);
    } else {
        if (a.channel_gate) launch_tokens_p<P, false, true>(bf16_io, D, a, grid, s);
        else                launch_tokens_p<P, false, false>(bf16_io, D, a, grid, s);
    }
}

hipError_t launch_decode_tokens(bool bf16_io, int D, const TokensArgs &a, hipStream_t s,
                                bool raw) {
    if ((long long)a.B * a.H <= 0 || a.n <= 0) return hipSuccess;
    constexpr int P = GDR_DECODE_PASSES;
    const long long per_head = D == 128 ? 128 / (Geom<128>::RPI * P) : 64 / (Geom<64>::RPI * P);
    const long long blocks = (long long)a.B * a.H * per_head;
    if (blocks >= (1LL << 31)) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks);
    launch_tokens_any<P>(bf16_io, D, a, grid, s, raw);
    return hipGetLastError();
}

hipError_t launch_decode_commit(int D, const TokensArgs &a, const int32_t *accepted,
                                hipStream_t s) {
    if ((long long)a.B * a.H <= 0 || a.n <= 0) return hipSuccess;
    const long long blocks = (long long)a.B * a.H * (D * D / 4096);
    if (blocks >= (1LL << 31)) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(256);
    if (D == 128) hipLaunchKernelGGL((commit_kernel<128>), grid, block, 0, s, a, accepted);
    else          hipLaunchKernelGGL((commit_kernel<64>), grid, block, 0, s, a, accepted);
    return hipGetLastError();
}

hipError_t launch_prefill_recurrent(bool bf16_io, int D, const PrefillArgs &a,
                                    hipStream_t s) {
    const long long blocks = (long long)a.N * a.H;
    if (blocks <= 0) return hipSuccess;
    // A fixed-length batch whose final state is wanted runs as the tokens of
    // a decode over its T tokens, from h0 (or zeros) into ht: the rows of a
    // state split over D / RPI workgroups (one pass each), so a thread
    // carries a quarter (D = 64) or a sixteenth (D = 128) of the state the
    // one-workgroup kernel below gives it, and a token's step is that much
    // shorter -- the latency of a short sequence.
    if (!a.cu_seqlens && !a.h0_slot && !a.ht_slot && a.ht && a.T > 0) {
        TokensArgs t{};
        t.init = a.h0;
        t.init_zero = a.h0 ? 0 : 1;
        t.q = a.q; t.k = a.k; t.v = a.v; t.g = a.g; t.beta = a.beta;
        t.slot = nullptr; t.pool = a.N; t.state = a.ht; t.ckpt = nullptr; t.o = a.o;
        t.B = a.N; t.n = a.T; t.H = a.H; t.scale = a.scale; t.channel_gate = a.channel_gate;
        t.xg = a.xg; t.xb = a.xb; t.gate_scale = a.gate_scale;
        const long long tb = blocks * (D == 128 ? 128 / Geom<128>::RPI : 64 / Geom<64>::RPI);
        if (tb >= (1LL << 31)) return hipErrorInvalidValue;
        launch_tokens_any<1>(bf16_io, D, t, dim3((unsigned)tb), s, a.xg != nullptr);
        return hipGetLastError();
    }
    dim3 grid((unsigned)blocks), block(256);
#define GDR_REC(TT, DD, RR)                                                                   \
    do {                                                                                      \
        if (a.channel_gate) hipLaunchKernelGGL((prefill_recurrent_kernel<TT, DD, RR, true>), grid, block, 0, s, a); \
        else                hipLaunchKernelGGL((prefill_recurrent_kernel<TT, DD, RR, false>), grid, block, 0, s, a); \
    } while (0)
    if (a.xg) {
        if (bf16_io) { if (D == 128) GDR_REC(bf16, 128, true);  else GDR_REC(bf16, 64, true); }
        else         { if (D == 128) GDR_REC(float, 128, true); else GDR_REC(float, 64, true); }
    } else {
        if (bf16_io) { if (D == 128) GDR_REC(bf16, 128, false);  else GDR_REC(bf16, 64, false); }
        else         { if (D == 128) GDR_REC(float, 128, false); else GDR_REC(float, 64, false); }
    }
#undef GDR_REC
    return hipGetLastError();
}

}  // namespace gdr
