// fa_decode.hip -- split-KV decode for gfx950: one query token per (batch,
// head) against a contiguous [B,H,L,d] bf16 KV cache (the KV cache of the
// attention-backend page).  The work is bound by HBM bandwidth: every cached
// key and value is read exactly once and reused by nothing.
//
// Phase 1 (split kernel): the cache of each (b, h) is cut into S contiguous
// chunks, one workgroup per chunk.  Each wave streams 16-byte pieces of
// consecutive keys (d/8 lanes per key, so one load instruction covers 1 KiB of
// contiguous cache), keeps U loads of K and of V in flight per lane, reduces
// the dot products with DPP inside each row of 16 lanes and runs the online
// softmax (running max, running sum, rescaled accumulator: Slovak page,
// section 2; Greek page, online-softmax section) in fp32.  The partial states
// of the lanes and waves are merged with the same rule, and the chunk writes
// its normalised output o_s and its log-sum-exp lse_s.
//
// Phase 2 (merge kernel): M = max_s lse_s, lse = M + ln sum_s exp(lse_s - M),
// O = sum_s exp(lse_s - lse) o_s, the online-softmax rescaling applied to
// whole chunks.
#include "fa_common.hpp"
#include "fa_internal.hpp"

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

template <int D>
__global__ void __launch_bounds__(DEC_THREADS)
decode_split_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
                    const __bf16* __restrict__ Vc, float* __restrict__ Opart,
                    float* __restrict__ LSEpart, int G, int L, int S, int chunk, float c) {
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
    const int k_begin = s * chunk;
    const int k_end = min(L, k_begin + chunk);

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

    const size_t hoff = (size_t)(bh / G) * (size_t)L * D;   // this query head's cache head
    const __bf16* Kh = Kc + hoff + 8 * dc;
    const __bf16* Vh = Vc + hoff + 8 * dc;

    float m = -INFINITY, l = 0.f;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;

    for (int base = k_begin + w * STEP; base < k_end; base += DEC_WAVES * STEP) {
        uint4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = base + u * KPL + slot;
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = kr[u];
            if (key < k_end) {
                kr[u] = load_stream16(Kh + (size_t)key * D);
                vr[u] = load_stream16(Vh + (size_t)key * D);
            }
        }
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
            dot = (LPK == 16) ? dpp_sum16(dot) : dpp_sum8(dot);
            x[u] = (base + u * KPL + slot < k_end) ? dot : -INFINITY;
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
        const size_t pidx = (size_t)bh * S + s;
        Opart[pidx * D + tid] = (ll > 0.f) ? oo[0] / ll : 0.f;
        if (tid == 0) LSEpart[pidx] = (ll > 0.f) ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
    }
}

// One wave per (b, h); lane t handles dims t and t + 64 (d = 128) or t (d = 64).
template <int D>
__global__ void __launch_bounds__(DEC_THREADS)
decode_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ LSEpart,
                    __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int S) {
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * DEC_WAVES + (threadIdx.x >> 6);
    if (bh >= BH) return;
    const float* lp = LSEpart + (size_t)bh * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float tot = 0.f;
    for (int s = 0; s < S; ++s) tot += __expf(lp[s] - Mu);
    const float lse = (tot > 0.f) ? Mu + __logf(tot) : -INFINITY;
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    for (int s = 0; s < S; ++s) {
        const float wgt = (tot > 0.f) ? __expf(lp[s] - lse) : 0.f;
        const float* op = Opart + ((size_t)bh * S + s) * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(wgt, op[lane + 64 * i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) O[(size_t)bh * D + lane + 64 * i] = (__bf16)acc[i];
    if (LSE != nullptr && lane == 0) LSE[bh] = lse;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
    const int BH = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)(BH * a.splits)), dim3(DEC_THREADS), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o_part, a.lse_part,
                       a.H / a.Hkv, a.L, a.splits, a.chunk, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)((BH + DEC_WAVES - 1) / DEC_WAVES)),
                       dim3(DEC_THREADS), 0, st, a.o_part, a.lse_part, (__bf16*)a.o, a.lse, BH, a.splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
    if ((long long)a.B * a.H * a.splits > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace fa
