// fa_decode.hip -- split-KV decode for gfx950: one query token per (batch,
// query head) against a bf16 KV cache of Hkv heads (the KV cache of the
// attention-backend page), either contiguous [B,Hkv,L,d] or paged (a pool of
// fixed-size pages and a block table per sequence, the PagedAttention layout
// that page describes).  The work is bound by HBM bandwidth: every cached key
// and value is read once per (b, cache head) on the grouped path, once per
// query head otherwise.
//
// Phase 1, per-head kernel (decode_split_kernel; H = Hkv, or groups larger
// than 32): the cache of each (b, h) is cut into S contiguous chunks, one
// workgroup per chunk.  Each wave streams 16-byte pieces of consecutive keys
// (d/8 lanes per key, so one load instruction covers 1 KiB of contiguous
// cache), keeps U loads of K and of V in flight per lane, reduces the dot
// products with DPP inside rows of 16 lanes and runs the online softmax
// (running max, running sum, rescaled accumulator: Slovak page, section 2;
// Greek page, online-softmax section) in fp32.  The partial states of the
// lanes and waves are merged with the same rule, and the chunk writes its
// normalised output o_s and its log-sum-exp lse_s.
//
// Phase 1, grouped kernels (2 <= H/Hkv <= 32; the choice between them is
// made by decode_small_group): decode_small_group_kernel for groups of 2 to
// 4, decode_group_kernel (MFMA) for the rest; see their own comments below.
//
// Phase 2 (merge kernel): M = max_s lse_s, lse = M + ln sum_s exp(lse_s - M),
// O = sum_s exp(lse_s - lse) o_s, the online-softmax rescaling applied to
// whole chunks.  With one chunk (S = 1) that is the identity, so the per-head
// and small-group kernels then write O and the LSE themselves and the merge
// is not launched.
#include "fa_common.hpp"
#include "fa_internal.hpp"

#include <type_traits>

namespace fa {

namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_UNROLL = 4;

// Merge (mb, lb, ob) into (ma, la, oa).
template <int NV>
__device__ __forceinline__ void merge_state(float& ma, float& la, float* oa, float mb, float lb,
                                            const float* ob) {
    const float mn = fmaxf(ma, mb);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float fa = exp2_fast(ma - mu), fb = exp2_fast(mb - mu);
    la = la * fa + lb * fb;
#pragma unroll
    for (int j = 0; j < NV; ++j) oa[j] = oa[j] * fa + ob[j] * fb;
    ma = mn;
}

// A value every lane of the wave reads from the same address of memory the
// kernel never writes (a block-table entry): read through the scalar data
// cache.  Scalar loads are counted apart from the vector loads, which retire
// in order, so waiting for the entry never waits for K/V loads in flight.
__device__ __forceinline__ int load_uniform(const int* p) {
    return *(const __attribute__((address_space(4))) int*)p;
}

template <int D, bool PAGED>
__global__ void __launch_bounds__(DEC_THREADS)
decode_split_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
                    const __bf16* __restrict__ Vc, float* __restrict__ Opart,
                    float* __restrict__ LSEpart, __bf16* __restrict__ Ofin, float* __restrict__ LSEfin,
                    int G, int L, int S, int chunk, float c, Paging pg) {
    constexpr int LPK = D / 8;           // lanes per key (8 bf16 each)
    constexpr int KPL = 64 / LPK;        // keys covered by one wave-wide load
    constexpr int U = DEC_UNROLL;
    constexpr int STEP = KPL * U;        // keys per wave per iteration

    __shared__ float sh_o[DEC_WAVES][D];
    __shared__ float sh_m[DEC_WAVES], sh_l[DEC_WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int slot = lane / LPK, dc = lane % LPK;
    const int s = blockIdx.x % S;
    const int bh = blockIdx.x / S;
    const int gkv = bh / G;                 // b * Hkv + cache head of this query head
    int Lb = L;                             // this sequence's cache length
    int b = 0, hk = 0;
    if constexpr (PAGED) {
        b = gkv / pg.Hkv;
        hk = gkv % pg.Hkv;
        Lb = min(max(pg.seq_lens[b], 0), L);
    }
    const int k_begin = s * chunk;
    const int k_end = min(Lb, k_begin + chunk);   // may be <= k_begin: an empty chunk

    // element offset of cached row `key` of this head, given (paged) the
    // block-table entry of its page; `ok` is false for a key on a page
    // outside the pool (such keys are skipped)
    auto row_of = [&](int key, int page, bool& ok) __attribute__((always_inline)) -> size_t {
        if constexpr (PAGED) {
            ok = page >= 0 && page < pg.num_pages;
            const size_t prow = (((size_t)(ok ? page : 0) * pg.Hkv + hk) << pg.ps_log2) +
                                (size_t)(key & ((1 << pg.ps_log2) - 1));
            return prow * D;
        } else {
            ok = true;
            return ((size_t)gkv * L + key) * D;
        }
    };
    // Block-table entry of the iteration at `base`, read one iteration ahead
    // so that the lookup is off the path of the K/V loads that depend on it.
    // An iteration's STEP keys start at a multiple of STEP (chunks are
    // multiples of 32 keys and STEP divides 32) and a page holds at least 32
    // keys, so they all lie in one page: one scalar read per wave.
    static_assert(32 % STEP == 0, "an iteration's keys lie in one page");
    auto fetch_page = [&](int base) __attribute__((always_inline)) -> int {
        const int kb = __builtin_amdgcn_readfirstlane(base);
        return (kb < k_end) ? load_uniform(pg.block_table + (size_t)b * pg.max_pages + (kb >> pg.ps_log2)) : -1;
    };

    // q, pre-multiplied by scale*log2(e), 8 dims per lane
    float qv[8];
    {
        const uint4 u = *reinterpret_cast<const uint4*>(Q + (size_t)bh * D + 8 * dc);
        const uint32_t* p = reinterpret_cast<const uint32_t*>(&u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qv[2 * j] = bf16_lo(p[j]) * c;
            qv[2 * j + 1] = bf16_hi(p[j]) * c;
        }
    }

    const __bf16* Kl = Kc + 8 * dc;         // this lane's 8 dims of any row
    const __bf16* Vl = Vc + 8 * dc;

    float m = -INFINITY, l = 0.f;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;

    int pg_next = 0;
    if constexpr (PAGED) pg_next = fetch_page(k_begin + w * STEP);
    for (int base = k_begin + w * STEP; base < k_end; base += DEC_WAVES * STEP) {
        uint4 kr[U], vr[U];
        bool live[U];
        const int pg_cur = pg_next;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = base + u * KPL + slot;
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = kr[u];
            live[u] = false;
            if (key < k_end) {
                const size_t r = row_of(key, pg_cur, live[u]);
                if (live[u]) {
                    kr[u] = load_stream16(Kl + r);
                    vr[u] = load_stream16(Vl + r);
                }
            }
        }
        if constexpr (PAGED) pg_next = fetch_page(base + DEC_WAVES * STEP);
        float x[U];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(&kr[u]);
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dot = fmaf(bf16_lo(p[j]), qv[2 * j], dot);
                dot = fmaf(bf16_hi(p[j]), qv[2 * j + 1], dot);
            }
            if constexpr (LPK == 8) {
                dot = dpp_sum8(dot);
            } else {
                dot = dpp_sum16(dot);
                if constexpr (LPK == 32) dot += __shfl_xor(dot, 16);   // d = 256: two rows per key
            }
            x[u] = live[u] ? dot : -INFINITY;
            mx = fmaxf(mx, x[u]);
        }
        const float mn = fmaxf(m, mx);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = exp2_fast(m - mu);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = exp2_fast(x[u] - mu);
            l += p;
            const uint32_t* vp = reinterpret_cast<const uint32_t*>(&vr[u]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[2 * j] = fmaf(p, bf16_lo(vp[j]), o[2 * j]);
                o[2 * j + 1] = fmaf(p, bf16_hi(vp[j]), o[2 * j + 1]);
            }
        }
    }

    // merge the KPL key slots of the wave (lanes dc, dc + LPK, ...)
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
        const float mb = __shfl_xor(m, off), lb = __shfl_xor(l, off);
        float ob[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ob[j] = __shfl_xor(o[j], off);
        merge_state<8>(m, l, o, mb, lb, ob);
    }
    if (slot == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sh_o[w][8 * dc + j] = o[j];
        if (dc == 0) {
            sh_m[w] = m;
            sh_l[w] = l;
        }
    }
    __syncthreads();
    if (tid < D) {
        float mm = sh_m[0], ll = sh_l[0];
        float oo[1] = {sh_o[0][tid]};
#pragma unroll
        for (int ww = 1; ww < DEC_WAVES; ++ww) {
            const float ob[1] = {sh_o[ww][tid]};
            merge_state<1>(mm, ll, oo, sh_m[ww], sh_l[ww], ob);
        }
        const float ov = (ll > 0.f) ? oo[0] / ll : 0.f;
        const float lv = (ll > 0.f) ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
        if (Ofin != nullptr) {          // one split: the final row
            Ofin[(size_t)bh * D + tid] = (__bf16)ov;
            if (tid == 0 && LSEfin != nullptr) LSEfin[bh] = lv;
        } else {
            const size_t pidx = (size_t)bh * S + s;
            Opart[pidx * D + tid] = ov;
            if (tid == 0) LSEpart[pidx] = lv;
        }
    }
}

// v += (v moved across the lanes of its row by the DPP control CTL), for
// every element of an array
template <int CTL, int N>
__device__ __forceinline__ void dpp_step_n(float* v) {
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), CTL, 0xF, 0xF, true));
}

// ---------------------------------------------------------------------------
// Grouped-query decode for small groups (GH = H/Hkv query heads per cache
// head, GH = 2, 3 or 4): the per-head kernel's streaming layout and online
// softmax, with the GH query heads of a cache head carried by the same lanes,
// so each cached key and value is loaded once for the group.  One workgroup
// per (batch, cache head, chunk).  The scores are bf16 dot2 products of the
// key with the unscaled query (a product of two bf16 values is exact in
// fp32), reduced over the key's lanes; scale*log2(e) (c > 0) is applied
// inside the exponent's FMA.  The value update is a bf16 dot2 over pairs of
// keys.
// ---------------------------------------------------------------------------
constexpr float kLazyRescale = 8.f;   // log2 of the largest term the sums may hold
template <int D, int GH, bool PAGED>
__global__ void __launch_bounds__(DEC_THREADS)
decode_small_group_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
                          const __bf16* __restrict__ Vc, float* __restrict__ Opart,
                          float* __restrict__ LSEpart, __bf16* __restrict__ Ofin, float* __restrict__ LSEfin,
                          int L, int S, int chunk, float c, Paging pg) {
    constexpr int LPK = D / 8;
    constexpr int KPL = 64 / LPK;
    constexpr int U = DEC_UNROLL;
    constexpr int STEP = KPL * U;

    __shared__ float sh_o[DEC_WAVES][GH][D];
    __shared__ float sh_m[DEC_WAVES][GH], sh_l[DEC_WAVES][GH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int slot = lane / LPK, dc = lane % LPK;
    const int s = blockIdx.x % S;
    const int gkv = blockIdx.x / S;         // b * Hkv + cache head
    int Lb = L;
    int b = 0, hk = 0;
    if constexpr (PAGED) {
        b = gkv / pg.Hkv;
        hk = gkv % pg.Hkv;
        Lb = min(max(pg.seq_lens[b], 0), L);
    }
    const int k_begin = s * chunk;
    const int k_end = min(Lb, k_begin + chunk);

    auto row_of = [&](int key, int page, bool& ok) __attribute__((always_inline)) -> size_t {
        if constexpr (PAGED) {
            ok = page >= 0 && page < pg.num_pages;
            const size_t prow = (((size_t)(ok ? page : 0) * pg.Hkv + hk) << pg.ps_log2) +
                                (size_t)(key & ((1 << pg.ps_log2) - 1));
            return prow * D;
        } else {
            ok = true;
            return ((size_t)gkv * L + key) * D;
        }
    };
    // block-table entry of the iteration at `base`: one page, one scalar read
    // per wave, one iteration ahead (as in decode_split_kernel)
    static_assert(32 % STEP == 0, "an iteration's keys lie in one page");
    auto fetch_page = [&](int base) __attribute__((always_inline)) -> int {
        const int kb = __builtin_amdgcn_readfirstlane(base);
        return (kb < k_end) ? load_uniform(pg.block_table + (size_t)b * pg.max_pages + (kb >> pg.ps_log2)) : -1;
    };

    // the GH query rows (query head gkv*GH + g), 8 packed bf16 dims per lane
    bf16x2 qp[GH][4];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
        const uint4 u = *reinterpret_cast<const uint4*>(Q + ((size_t)gkv * GH + g) * D + 8 * dc);
        qp[g][0] = __builtin_bit_cast(bf16x2, u.x);
        qp[g][1] = __builtin_bit_cast(bf16x2, u.y);
        qp[g][2] = __builtin_bit_cast(bf16x2, u.z);
        qp[g][3] = __builtin_bit_cast(bf16x2, u.w);
    }

    const __bf16* Kl = Kc + 8 * dc;
    const __bf16* Vl = Vc + 8 * dc;

    float m[GH], l[GH], o[GH][8];
#pragma unroll
    for (int g = 0; g < GH; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
    }

    int pg_next = 0;
    if constexpr (PAGED) pg_next = fetch_page(k_begin + w * STEP);
    for (int base = k_begin + w * STEP; base < k_end; base += DEC_WAVES * STEP) {
        uint4 kr[U], vr[U];
        bool live[U];
        const int pg_cur = pg_next;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = base + u * KPL + slot;
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = kr[u];
            live[u] = false;
            if (key < k_end) {
                const size_t r = row_of(key, pg_cur, live[u]);
                if (live[u]) {
                    kr[u] = load_stream16(Kl + r);
                    vr[u] = load_stream16(Vl + r);
                }
            }
        }
        if constexpr (PAGED) pg_next = fetch_page(base + DEC_WAVES * STEP);
        // scores: the dot2 partial sums of every (head, key) first, then the
        // reductions over the key's lanes one step at a time across all of
        // them, so consecutive DPP adds are independent
        float x[GH][U];
#pragma unroll
        for (int g = 0; g < GH; ++g)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = 0.f;
                dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[u].x), qp[g][0], dot, false);
                dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[u].y), qp[g][1], dot, false);
                dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[u].z), qp[g][2], dot, false);
                x[g][u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[u].w), qp[g][3], dot, false);
            }
        dpp_step_n<0xB1, GH * U>(&x[0][0]);      // [1,0,3,2]
        dpp_step_n<0x4E, GH * U>(&x[0][0]);      // [2,3,0,1]
        dpp_step_n<0x141, GH * U>(&x[0][0]);     // half mirror
        if constexpr (LPK >= 16) dpp_step_n<0x140, GH * U>(&x[0][0]);    // row mirror
        if constexpr (LPK == 32) {     // d = 256: two rows per key
#pragma unroll
            for (int g = 0; g < GH; ++g)
#pragma unroll
                for (int u = 0; u < U; ++u) x[g][u] += __shfl_xor(x[g][u], 16);
        }
        float mxs[GH], mu[GH];
        bool grow = false;
#pragma unroll
        for (int g = 0; g < GH; ++g) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[g][u] = live[u] ? x[g][u] : -INFINITY;
                mx = fmaxf(mx, x[g][u]);
            }
            mxs[g] = mx * c;
            grow = grow || mxs[g] > m[g] + kLazyRescale;
        }
        // m is a reference value, raised only when a score exceeds it by more
        // than 2^kLazyRescale (decided per wave, so the branch is uniform); l
        // and o are sums of 2^(c*x - m) for any such reference
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const float mn = fmaxf(m[g], mxs[g]);
                const float alpha = exp2_fast(m[g] - ((mn == -INFINITY) ? 0.f : mn));
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] *= alpha;
            }
        }
#pragma unroll
        for (int g = 0; g < GH; ++g) mu[g] = (m[g] == -INFINITY) ? 0.f : m[g];
        // values, two keys at a time: v_perm gathers dim j of keys u and u+1
        // into one bf16 pair, p of the two keys is packed to bf16 (as the
        // PV products of the forward use it) and o_j += dot2(p, v_j); the
        // running sum adds the same rounded p
#pragma unroll
        for (int u = 0; u < U; u += 2) {
            const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vr[u]);
            const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vr[u + 1]);
            bf16x2 vv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vv[2 * j] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(v1[j], v0[j], 0x05040100u));
                vv[2 * j + 1] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(v1[j], v0[j], 0x07060302u));
            }
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const uint32_t pp = pack_bf16x2(exp2_fast(fmaf(x[g][u], c, -mu[g])),
                                                exp2_fast(fmaf(x[g][u + 1], c, -mu[g])));
                l[g] = sum_bf16x2(pp, l[g]);
                const bf16x2 pb = __builtin_bit_cast(bf16x2, pp);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] = __builtin_amdgcn_fdot2_f32_bf16(vv[j], pb, o[g][j], false);
            }
        }
    }

    // merge the KPL key slots of the wave, then the waves through LDS
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GH; ++g) {
            const float mb = __shfl_xor(m[g], off), lb = __shfl_xor(l[g], off);
            float ob[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) ob[j] = __shfl_xor(o[g][j], off);
            merge_state<8>(m[g], l[g], o[g], mb, lb, ob);
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int g = 0; g < GH; ++g) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sh_o[w][g][8 * dc + j] = o[g][j];
            if (dc == 0) {
                sh_m[w][g] = m[g];
                sh_l[w][g] = l[g];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < GH * D; i += DEC_THREADS) {
        const int g = i / D, dd = i % D;
        float mm = sh_m[0][g], ll = sh_l[0][g];
        float oo[1] = {sh_o[0][g][dd]};
#pragma unroll
        for (int ww = 1; ww < DEC_WAVES; ++ww) {
            const float ob[1] = {sh_o[ww][g][dd]};
            merge_state<1>(mm, ll, oo, sh_m[ww][g], sh_l[ww][g], ob);
        }
        const size_t hq = (size_t)gkv * GH + g;        // query head (b*H + h)
        const float ov = (ll > 0.f) ? oo[0] / ll : 0.f;
        const float lv = (ll > 0.f) ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
        if (Ofin != nullptr) {          // one split: the final row
            Ofin[hq * D + dd] = (__bf16)ov;
            if (dd == 0 && LSEfin != nullptr) LSEfin[hq] = lv;
        } else {
            const size_t pidx = hq * S + s;
            Opart[pidx * D + dd] = ov;
            if (dd == 0) LSEpart[pidx] = lv;
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped-query decode: the G <= 32 query heads that share a cache head are
// processed together, so each cached key and value is read from HBM once per
// group instead of once per query head.  The heads are the rows of a small
// matrix product: with q^T of the group as the B operand (G columns, padded
// to 32 with zeros), S^T = K q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_bf16 exactly as in the forward kernel, with the keys as
// the streamed dimension.  Each wave is an independent unit of work -- one
// (batch, cache head, key chunk) -- with its own double-buffered 32-key K and
// V tiles in LDS filled by buffer DMA, so no workgroup barrier is needed.  The
// online softmax (lazy rescaling as in the forward) runs per head column; the
// unit writes the normalised partial o_s and lse_s of its G heads, and the
// merge kernel below combines the chunks.
// ---------------------------------------------------------------------------
constexpr int DG_BC = 32;          // keys per tile

// s_waitcnt on vmcnt only (expcnt and lgkmcnt at their maximum)
#define DG_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))
static_assert(kDecodeMaxGroup <= 32, "one 32-column MFMA block of heads per unit");

// waves (units) per workgroup: the d = 256 tiles are twice as large
template <int D>
constexpr int dg_waves() { return D == 256 ? 2 : 4; }

template <int D, bool PAGED>
__global__ void __launch_bounds__(64 * dg_waves<D>())
decode_group_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
                    const __bf16* __restrict__ Vc, float* __restrict__ Opart,
                    float* __restrict__ LSEpart, int G, int L, int S, int chunk, int units,
                    float c /* scale * log2(e) */, Paging pg) {
    constexpr int ROWB = 2 * D;             // bytes per cached row
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int TILEB = DG_BC * ROWB;     // one K (or V) tile of one wave
    constexpr int SEGS = TILEB / 1024;      // 1 KiB copy segments per tile
    constexpr int RPS = 1024 / ROWB;        // rows per segment
    constexpr float TAU = 8.f;              // lazy-rescale threshold, log2 units

    // per-wave tile buffers; four separate LDS objects so that the copies into
    // one buffer pair do not make the reads of the other wait
    __shared__ __attribute__((aligned(1024))) char kb0[dg_waves<D>()][TILEB];
    __shared__ __attribute__((aligned(1024))) char kb1[dg_waves<D>()][TILEB];
    __shared__ __attribute__((aligned(1024))) char vb0[dg_waves<D>()][TILEB];
    __shared__ __attribute__((aligned(1024))) char vb1[dg_waves<D>()][TILEB];

    // w is the same in every lane; saying so keeps the LDS destinations of the
    // copies (M0) in scalar registers without a per-lane loop
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int unit = blockIdx.x * dg_waves<D>() + w;
    if (unit >= units) return;              // no barrier below: waves are independent
    const int s = unit % S;
    const int gkv = unit / S;               // b * Hkv + cache head
    int Lb = L;                             // this sequence's cache length
    int b = 0, hk = 0;
    if constexpr (PAGED) {
        b = gkv / pg.Hkv;
        hk = gkv % pg.Hkv;
        Lb = min(max(pg.seq_lens[b], 0), L);
    }
    const int k_begin = s * chunk;          // chunk is a multiple of 32, so a paged
    const int k_end = min(Lb, k_begin + chunk);   // tile never straddles two pages
    const int ntile = k_end > k_begin ? (k_end - k_begin + DG_BC - 1) / DG_BC : 0;

    // q^T of the group as the B operand: column l32 is query head gkv*G + l32
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (l32 < G)
            u = *reinterpret_cast<const uint4*>(Q + ((size_t)gkv * G + l32) * D + 16 * ks + 8 * g);
        qf[ks] = as_bf16x8(u);
    }

    // Contiguous: one resource over the cache head (L * ROWB bytes < 2^32,
    // checked by the host).  Paged: one resource per tile over its 32 rows of
    // a page, empty when the page index lies outside the pool (its loads then
    // read zeros and its keys are masked).
    const size_t hoff = (size_t)gkv * (size_t)L * D;
    __amdgpu_buffer_rsrc_t k_rs = make_rsrc(Kc + hoff, (uint32_t)L * ROWB);
    __amdgpu_buffer_rsrc_t v_rs = make_rsrc(Vc + hoff, (uint32_t)L * ROWB);
    // Paged: the block-table entries of this unit's pages, 64 at a time, one
    // per lane (lane i holds page pw0 + i of the sequence).  A tile takes its
    // entry with readlane, so no table read (and no wait for it, which would
    // also wait for the copies in flight) sits between two tiles; a new window
    // is read once every 64 pages.
    int pwin = -1, pw0 = 0;
    auto load_window = [&](int first) __attribute__((always_inline)) {
        pw0 = first;
        const int pidx = first + lane;
        pwin = (pidx <= ((k_end - 1) >> pg.ps_log2)) ? pg.block_table[(size_t)b * pg.max_pages + pidx] : -1;
        DG_WAIT_VMCNT0();   // here, so the tiles that follow need not wait for it
    };
    if constexpr (PAGED) {
        if (ntile > 0) load_window(k_begin >> pg.ps_log2);
    }
    auto page_of = [&](int k0, bool& ok) __attribute__((always_inline)) -> size_t {
        const int pidx = k0 >> pg.ps_log2;
        if (pidx - pw0 >= 64) load_window(pidx);
        const int page = __builtin_amdgcn_readlane(pwin, pidx - pw0);
        ok = page >= 0 && page < pg.num_pages;
        return ((((size_t)(ok ? page : 0) * pg.Hkv + hk) << pg.ps_log2) +
                (size_t)(k0 & ((1 << pg.ps_log2) - 1))) * D;
    };
    // copy the 32 rows of tile t; rows past the live keys repeat the last live
    // row (masked for K, weighted by 0 for V), so no unwritten cache row is read
    bool ok_issued = true;                   // paged: the last issued tile's page is in the pool
    auto issue = [&](int t, char* kdst, char* vdst) __attribute__((always_inline)) {
        const int k0 = k_begin + t * DG_BC;
        int rbase = k0;                      // row of the resource where the tile starts
        if constexpr (PAGED) {
            bool ok;
            const size_t off = page_of(k0, ok);
            ok_issued = ok;
            k_rs = make_rsrc(Kc + off, ok ? (uint32_t)(DG_BC * ROWB) : 0u);
            v_rs = make_rsrc(Vc + off, ok ? (uint32_t)(DG_BC * ROWB) : 0u);
            rbase = 0;
        }
#pragma unroll
        for (int seg = 0; seg < SEGS; ++seg) {
            const int row = seg * RPS + lane / CPR;
            const int pc = lane % CPR;
            const uint32_t grow = (uint32_t)(rbase + min(row, k_end - 1 - k0)) * ROWB;
            b2lds16(k_rs, grow + 16 * (pc ^ k_swz<D>(row)), kdst + seg * 1024);
            b2lds16(v_rs, grow + 16 * (pc ^ v_swz<D>(row)), vdst + seg * 1024);
        }
    };

    // LDS offsets as in the forward: K rows read one chunk per lane, V^T read
    // with the transposing 8-byte read
    int k_off[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k_off[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ k_swz<D>(l32));
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int vsw = v_swz<D>(vr) >> 2;
    int v_off[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) v_off[mb] = vr * ROWB + 16 * (4 * (mb ^ vsw) + (vc >> 3)) + 2 * (vc & 7);

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_ref = -INFINITY, l_run = 0.f;

    auto step = [&](int t, const char* Ks, const char* Vs, char* kn, char* vn) __attribute__((always_inline)) {
        // this tile's copies have landed, and this wave's reads of the other
        // buffer pair (the previous tile) are complete before it is refilled
        const bool ok_t = ok_issued;         // page of this tile (issued a step earlier)
        __builtin_amdgcn_s_waitcnt(0);
        if (t + 1 < ntile) issue(t + 1, kn, vn);
        // S^T = K q^T: keys x heads; lane holds head l32, keys 8(r/4) + 4g + r%4
        f32x16 st = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            st = mfma_bf16(*reinterpret_cast<const bf16x8*>(Ks + k_off[ks]), qf[ks], st);
        int live_keys = k_end - (k_begin + t * DG_BC);
        if (PAGED && !ok_t) live_keys = 0;
        const int lim = live_keys - 1 - 4 * g;   // last live key slot of this lane
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            st[r] = (8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : st[r];
            mx = fmaxf(mx, st[r]);
        }
        mx = xor32_max(mx) * c;
        if (__any(mx > m_ref + TAU)) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = exp2_fast(m_ref - m_new);   // 0 on the first tile
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t pk[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float p0 = exp2_fast(fmaf(st[8 * h + j], c, -m_use));
                const float p1 = exp2_fast(fmaf(st[8 * h + j + 1], c, -m_use));
                pk[j / 2] = pack_bf16x2(p0, p1);
                psum = sum_bf16x2(pk[j / 2], psum);
            }
            pb[h] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
        l_run += psum;
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
                const uint2 lo = lds_read_tr16x4(Vs + (16 * ks) * ROWB + v_off[mb]);
                const uint2 hi = lds_read_tr16x4(Vs + (16 * ks + 8) * ROWB + v_off[mb]);
                oacc[mb] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[ks], oacc[mb]);
            }
    };

    if (ntile > 0) issue(0, kb0[w], vb0[w]);
    for (int t = 0; t < ntile; t += 2) {
        step(t, kb0[w], vb0[w], kb1[w], vb1[w]);
        if (t + 1 < ntile) step(t + 1, kb1[w], vb1[w], kb0[w], vb0[w]);
    }

    // normalised partial of each real head of the group
    const float l_tot = xor32_sum(l_run);
    if (l32 < G) {
        const size_t pidx = ((size_t)gkv * G + l32) * S + s;
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        float* orow = Opart + pidx * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                *reinterpret_cast<float4*>(orow + 32 * mb + 8 * rb + 4 * g) =
                    make_float4(oacc[mb][4 * rb] * inv, oacc[mb][4 * rb + 1] * inv,
                                oacc[mb][4 * rb + 2] * inv, oacc[mb][4 * rb + 3] * inv);
        if (g == 0) LSEpart[pidx] = (l_tot > 0.f) ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
    }
}

// One wave per (b, h).  The splits' LSEs are spread over the lanes (lane j
// holds split j, j + 64, ...) and reduced across the wave, so the statistics
// cost one load per 64 splits rather than a chain of dependent loads; each
// lane then accumulates dims lane, lane + 64, ... of O, loading the partial
// rows of eight splits before combining them.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
__global__ void __launch_bounds__(DEC_THREADS)
decode_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ LSEpart,
                    __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int S) {
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * DEC_WAVES + (threadIdx.x >> 6);
    if (bh >= BH) return;
    const float* lp = LSEpart + (size_t)bh * S;
    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
    M = wave_max(M);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float tot = 0.f;
    for (int s = lane; s < S; s += 64) tot += __expf(lp[s] - Mu);
    tot = wave_sum(tot);
    const float lse = (tot > 0.f) ? Mu + __logf(tot) : -INFINITY;
    constexpr int PER = D / 64;
    // partial rows loaded before they are combined: 64 registers' worth
    // (64, 32, 16 rows at d = 64, 128, 256), then blocks of 8, then single
    // rows, so that 64 splits take two load rounds at d = 128, not eight
    constexpr int U = 64 / PER;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    const float* orow = Opart + (size_t)bh * S * D + lane;
    // rows s0 + j .. s0 + j + R - 1, in split order
    auto block = [&](auto R, int s0, int j, float wl) __attribute__((always_inline)) {
        float v[decltype(R)::value][PER];
#pragma unroll
        for (int u = 0; u < decltype(R)::value; ++u)
#pragma unroll
            for (int i = 0; i < PER; ++i) v[u][i] = orow[(size_t)(s0 + j + u) * D + 64 * i];
#pragma unroll
        for (int u = 0; u < decltype(R)::value; ++u) {
            const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j + u));
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = fmaf(wu, v[u][i], acc[i]);
        }
    };
    for (int s0 = 0; s0 < S; s0 += 64) {
        // weight of split s0 + lane; split s0 + j's weight is read from lane j
        const float wl = (s0 + lane < S && tot > 0.f) ? __expf(lp[s0 + lane] - lse) : 0.f;
        const int n = min(64, S - s0);
        int j = 0;
        for (; j + U <= n; j += U) block(std::integral_constant<int, U>{}, s0, j, wl);
        for (; j + 8 <= n; j += 8) block(std::integral_constant<int, 8>{}, s0, j, wl);
        for (; j < n; ++j) block(std::integral_constant<int, 1>{}, s0, j, wl);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) O[(size_t)bh * D + lane + 64 * i] = (__bf16)acc[i];
    if (LSE != nullptr && lane == 0) LSE[bh] = lse;
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeArgs& a) {
    const int BH = a.B * a.H;
    const int G = a.H / a.Hkv;
    hipStream_t st = (hipStream_t)a.stream;
    // With one split each partial already is the final row: the per-head
    // and small-group kernels then write O (bf16) and the LSE themselves --
    // the same values the merge would (its weight for the only split is
    // e^0 = 1) -- and the merge launch is skipped.  The MFMA grouped kernel,
    // which serves small batches with many splits, always writes partials
    // (a direct-store path there measured 3% slower at batch 1).
    bool direct = a.splits == 1;
    __bf16* ofin = direct ? (__bf16*)a.o : nullptr;
    float* lfin = direct ? a.lse : nullptr;
    if (decode_small_group(a.B, a.H, a.Hkv) != 0) {
        const dim3 grid((unsigned)(a.B * a.Hkv * a.splits));
        if (G == 2) {
            hipLaunchKernelGGL((decode_small_group_kernel<D, 2, PAGED>), grid, dim3(DEC_THREADS), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o_part,
                               a.lse_part, ofin, lfin, a.L, a.splits, a.chunk, a.scale * kLog2e, a.paging);
        } else if (G == 3) {
            hipLaunchKernelGGL((decode_small_group_kernel<D, 3, PAGED>), grid, dim3(DEC_THREADS), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o_part,
                               a.lse_part, ofin, lfin, a.L, a.splits, a.chunk, a.scale * kLog2e, a.paging);
        } else {
            hipLaunchKernelGGL((decode_small_group_kernel<D, 4, PAGED>), grid, dim3(DEC_THREADS), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o_part,
                               a.lse_part, ofin, lfin, a.L, a.splits, a.chunk, a.scale * kLog2e, a.paging);
        }
    } else if (decode_group_path(a.B, a.H, a.Hkv)) {
        const int units = a.B * a.Hkv * a.splits;
        constexpr int WV = dg_waves<D>();
        hipLaunchKernelGGL((decode_group_kernel<D, PAGED>), dim3((unsigned)((units + WV - 1) / WV)),
                           dim3(64 * WV), 0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                           a.o_part, a.lse_part, G, a.L, a.splits, a.chunk, units, a.scale * kLog2e, a.paging);
        direct = false;
    } else {
        hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3((unsigned)(BH * a.splits)), dim3(DEC_THREADS), 0,
                           st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o_part, a.lse_part,
                           ofin, lfin, G, a.L, a.splits, a.chunk, a.scale * kLog2e, a.paging);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)((BH + DEC_WAVES - 1) / DEC_WAVES)),
                       dim3(DEC_THREADS), 0, st, a.o_part, a.lse_part, (__bf16*)a.o, a.lse, BH, a.splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
    if ((long long)a.B * a.H * a.splits > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.paging.block_table != nullptr) {
        if (a.d == 256) return launch_d<256, true>(a);
        return a.d == 64 ? launch_d<64, true>(a) : launch_d<128, true>(a);
    }
    if (a.d == 256) return launch_d<256, false>(a);
    return a.d == 64 ? launch_d<64, false>(a) : launch_d<128, false>(a);
}

}  // namespace fa
