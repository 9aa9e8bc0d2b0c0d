// fa_fwd.hip -- fused exact-attention forward for gfx950.
//
// One workgroup owns one tile of BR query rows of one (batch, head) and
// streams that head's K/V tiles through LDS, keeping the running row maximum,
// the running sum of exponentials and the unnormalised output in registers
// (online softmax: "FlashAttention (EL)", sections on tiling and on online
// softmax; "Flash Attention: Ako transformery ...", section 2).  QK^T,
// masking, softmax and PV are fused; only O and the per-row LSE are written
// (same Greek page, section on fusing all operations into one kernel).  Work
// is split over query tiles as well as heads so that small-batch long
// sequences fill the chip ("Flash Attention uitgelegd", FA2 section on
// parallelism over the sequence length).
//
// bf16 path (d = 64, 128 or 256): four waves, 32 query rows each.  Key tiles
// of BC = 64 keys at d = 64 (four workgroups per CU), 32 keys at d = 128
// (three per CU) and at d = 256 (two per CU, whose accumulators are twice as
// large).  Per key tile a wave computes S^T = K Q^T (keys x queries) with
// v_mfma_f32_32x32x16_bf16: K comes from LDS, Q^T stays in registers for the
// whole kernel.  In the C layout each lane then holds one query row and 16
// of the tile's keys, so row max and row sum are in-lane work plus one
// exchange with lane ^ 32.  The probabilities,
// rounded to bf16, are already a valid B operand of O^T += V^T P^T; the V^T A
// operand is read from the row-major V tile with the transposing LDS read.
// O^T again gives each lane one query row.  K and V tiles are copied
// global -> LDS by buffer DMA without passing through registers,
// double-buffered, and a fixed instruction schedule keeps LDS operand reads
// ahead of the MFMAs.  The scale is folded into the exp2 argument, the
// reference max is only raised when a tile's max exceeds it by more than 8 in
// log2 units (exact: the same reference is used for the numerator and the
// denominator), and O is normalised once at the end (the FA2 point about
// minimising non-matmul work).  With grouped-query attention (Hkv < H K/V
// heads) query head h reads K/V head h / (H / Hkv).
//
// fp32 path: v_mfma_f32_32x32x2_f32 with BC = 32 (V needs no transpose
// because each fp32 K-slot holds a single key), one workgroup per 32 query
// rows whose four waves split the key tiles and merge their partial results
// at the end (see fwd_f32_kernel).
//
// The bf16 kernel template lives in fa_fwd_kernel.hpp; this file holds the
// fp32 kernel and the launchers.
#include "fa_fwd_kernel.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

// fp32 path.  One workgroup per 32 query rows of one (b, h).  Its four waves
// split the key tiles -- wave w takes tiles w, w + 4, w + 8, ... -- each with
// the 32 query rows, its own LDS tile and its own online softmax, so the loop
// has no barrier.  At the end the four partial results (row max m, row sum l
// and the unnormalised O of each wave) are combined through LDS with the
// online-softmax merge rule: O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w
// with M = max_w m_w.  A 128-token head then runs on four CUs, each wave on
// one tile, instead of one CU whose waves each walk all four tiles.
constexpr int F32_BR = 32;      // query rows per workgroup
constexpr int F32_NW = FWD_THREADS / 64;   // waves splitting the key tiles

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(FWD_THREADS)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
               const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
               int BH, int G, int N, int nqt, float c) {
    constexpr int BR = F32_BR, BC = FWD_BC32, NW = F32_NW;
    constexpr int KS = D + 1;      // odd stride: column reads hit distinct banks
    constexpr int VS = D;
    constexpr int WTILE = BC * KS + BC * VS;       // floats of one wave's K and V tiles
    constexpr int CPL = BC * D / 4 / 64;           // 16-byte chunks per lane per tile
    constexpr int OS = D + 4;                      // row stride of the partial outputs
    static_assert(BR == BC, "the causal diagonal is one tile");
    static_assert(NW * BR * OS + 2 * NW * BR <= NW * WTILE, "the partials fit the tile space");

    __shared__ __attribute__((aligned(16))) float smem[NW * WTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    float* Ks = smem + w * WTILE;                  // this wave's tiles
    float* Vs = Ks + BC * KS;

    int bh, qt;
    fwd_tile_of(blockIdx.x, BH, G, nqt, CAUSAL, bh, qt);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const size_t kvoff = (size_t)(bh / G) * (size_t)N * D;
    const float* Qh = Q + hoff;
    const float* Kh = K + kvoff;
    const float* Vh = V + kvoff;

    // K-step ks of S^T = K Q^T takes dims ks (K-slot 0, lanes 0-31) and
    // ks + D/2 (K-slot 1, lanes 32-63): each lane holds one contiguous half
    // of its query row, loaded 16 bytes at a time
    const int qrow = q0 + l32;
    float qf[D / 2];
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qrow < N) u = *reinterpret_cast<const float4*>(Qh + (size_t)qrow * D + (D / 2) * g + 4 * j);
        qf[4 * j] = u.x;
        qf[4 * j + 1] = u.y;
        qf[4 * j + 2] = u.z;
        qf[4 * j + 3] = u.w;
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;

    // The wave's next tile is loaded into registers while the current one is
    // computed, and stored to its LDS tile after it.
    float4 kk[CPL], vv[CPL];
    auto load = [&](int kt) __attribute__((always_inline)) {
        const int kv0 = kt * BC;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            const int row = ch / (D / 4), c4 = ch % (D / 4);
            kk[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            vv[i] = kk[i];
            if (kv0 + row < N) {
                kk[i] = *reinterpret_cast<const float4*>(Kh + (size_t)(kv0 + row) * D + 4 * c4);
                vv[i] = *reinterpret_cast<const float4*>(Vh + (size_t)(kv0 + row) * D + 4 * c4);
            }
        }
    };
    if (w < nkt) load(w);
    for (int kt = w; kt < nkt; kt += NW) {
        const int kv0 = kt * BC;
        // Only this wave touches its tiles, and a wave's LDS operations run in
        // order, so the previous tile's reads are done before these writes
        // and the writes before the reads below.
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            const int row = ch / (D / 4), c4 = ch % (D / 4);
            float* kd = Ks + row * KS + 4 * c4;
            kd[0] = kk[i].x; kd[1] = kk[i].y; kd[2] = kk[i].z; kd[3] = kk[i].w;
            *reinterpret_cast<float4*>(Vs + row * VS + 4 * c4) = vv[i];
        }
        if (kt + NW < nkt) load(kt + NW);

        f32x16 s = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) s = mfma_f32(Ks[l32 * KS + ks + (D / 2) * g], qf[ks], s);

        if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > q0)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= N || (CAUSAL && key > qrow)) s[r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = xor32_max(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_fast(fmaf(s[r], c, -m_use));
            psum += s[r];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
            // K-slot r of this lane = key 8*(r/4) + 4*g + r%4, matching C register r of S^T
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * g + (r & 3);
                oacc[mb] = mfma_f32(Vs[key * VS + 32 * mb + l32], s[r], oacc[mb]);
            }
        }
    }

    // Merge the waves' partial results.  A wave without tiles (or whose keys
    // are all hidden) has m = -inf, l = 0 and O = 0 and gets weight 0.
    const float l_tot = xor32_sum(l_run);
    __syncthreads();                               // every wave is done with its tiles
    float* Op = smem;                              // [NW][BR][OS] unnormalised O
    float* Mp = smem + NW * BR * OS;               // [NW][BR] row max, log2 units
    float* Lp = Mp + NW * BR;                      // [NW][BR] row sum
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<float4*>(Op + (w * BR + l32) * OS + 32 * mb + 8 * rb + 4 * g) =
                make_float4(oacc[mb][4 * rb], oacc[mb][4 * rb + 1], oacc[mb][4 * rb + 2], oacc[mb][4 * rb + 3]);
    if (g == 0) {
        Mp[w * BR + l32] = m_run;
        Lp[w * BR + l32] = l_tot;
    }
    __syncthreads();
    // 8 threads per row, each 4 columns at a time: a row is written with
    // 16-byte stores by consecutive lanes.
    constexpr int TPR = FWD_THREADS / BR;
    const int r = tid / TPR, part = tid % TPR;
    const int row = q0 + r;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, Mp[v * BR + r]);
    float a[NW], L = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const float mv = Mp[v * BR + r];
        a[v] = (mv == -INFINITY) ? 0.f : exp2_fast(mv - M);
        L = fmaf(a[v], Lp[v * BR + r], L);
    }
    if (row < N) {
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        float* orow = O + (size_t)bh * N * D + (size_t)row * D;
#pragma unroll
        for (int j = 0; j < D / (4 * TPR); ++j) {
            const int col = 4 * (part + TPR * j);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float4 p = *reinterpret_cast<const float4*>(Op + (v * BR + r) * OS + col);
                acc.x = fmaf(a[v], p.x, acc.x);
                acc.y = fmaf(a[v], p.y, acc.y);
                acc.z = fmaf(a[v], p.z, acc.z);
                acc.w = fmaf(a[v], p.w, acc.w);
            }
            *reinterpret_cast<float4*>(orow + col) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        }
        if (part == 0)
            LSE[(size_t)bh * N + row] = (L > 0.f) ? M * kLn2 + __logf(L) : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16(const FwdArgs& a) {
    const int BH = a.B * a.H;
    const int nqt = (a.N + FWD_BR - 1) / FWD_BR;
    const dim3 grid((unsigned)(nqt * BH)), block(FWD_THREADS);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_BF16>), grid, block, 0, (hipStream_t)a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse, BH,
                       a.H / a.Hkv, a.N, nqt, a.scale * kLog2e, nullptr);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs& a) {
    const int BH = a.B * a.H;
    const int nqt = (a.N + F32_BR - 1) / F32_BR;
    const dim3 grid((unsigned)(nqt * BH)), block(FWD_THREADS);
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, (hipStream_t)a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, BH,
                       a.H / a.Hkv, a.N, nqt, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(const FwdArgs& a) {
    if constexpr (D != 256) {   // fp32 inputs: d = 64 and 128 only (the host rejects d = 256)
        if (!a.in_bf16) return a.causal ? launch_f32<D, true>(a) : launch_f32<D, false>(a);
    }
    if (a.out_bf16) return a.causal ? launch_bf16<D, true, true>(a) : launch_bf16<D, false, true>(a);
    return a.causal ? launch_bf16<D, true, false>(a) : launch_bf16<D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
    if ((long long)((a.N + F32_BR - 1) / F32_BR) * a.B * a.H > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.d == 256) return dispatch_d<256>(a);
    return a.d == 64 ? dispatch_d<64>(a) : dispatch_d<128>(a);
}

}  // namespace fa
