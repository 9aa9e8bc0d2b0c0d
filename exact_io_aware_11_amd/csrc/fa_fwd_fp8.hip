// fa_fwd_fp8.hip -- exact-attention forward on fp8 (e4m3) inputs for gfx950.
//
// Same algorithm as the bf16 forward (tiling and online softmax: "FlashAttention
// (EL)", sections on tiling and on online softmax; the FP8 support named on
// "Flash Attention uitgelegd", FA3 section): one workgroup of four waves per
// 128 query rows, 64-key K/V tiles streamed through LDS by buffer DMA, double
// buffered, S and O accumulated in fp32.  The products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit block scales), twice the
// bf16 rate.  The caller passes per-tensor dequantisation factors for Q, K and
// V; they are folded into the exponent scale and the final normalisation.
//
// Probabilities.  P enters the second product as e4m3 too.  To keep its
// rounding relative (3 mantissa bits) rather than absolute, the reference max
// is the tile-by-tile running max rounded up to an integer in base-2 units:
// every probability is then at most 1 and every rescale an exact power of two.
// P is scaled by 2^8 before rounding, so values down to 2^-14 stay normal in
// e4m3.  The row sum adds the unrounded fp32 values, so the LSE is that of the
// inputs; the rounding of P is the only approximation beyond fp32
// accumulation.
//
// Operand layout.  For S^T = K Q^T each lane holds 32 bytes of one K row (the
// A operand) and the same 32 dims of its query row (the B operand); A and B
// use the same K-slot order, whatever the hardware's, so any consistent split
// of the dims works.  For O^T += V^T P^T the B operand is P straight from the
// S accumulator: lane (query, g) holds the 32 keys kb*32 + 8q + 4g + t
// (kb, q, t < 2, 4, 4), packed in that order.  V arrives transposed ([d, N]
// per head), and each 64-key V^T tile is copied with 4-byte DMA into a key
// order in which the same 32 keys sit contiguous at byte 32g of every dim row,
// so the A operand is two 16-byte LDS reads.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int F8_BR = 128;       // query rows per workgroup (4 waves x 32)
constexpr int F8_BC = 64;        // keys per K/V tile
constexpr int F8_THREADS = 256;

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
    // cbsz = blgp = 0: both operands e4m3; block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join8(uint4 lo, uint4 hi) {
    i32x8 r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// four e4m3 values (round to nearest even) in one word, a first
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c2, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c2, d, lo, true);
}

// source dword (4 keys) of the 64-key tile row that belongs at logical dword
// u of the LDS row: u = 8g + 4kb + q holds keys kb*32 + 8q + 4g .. +3
__device__ __forceinline__ int vt_src_dword(int u) { return ((u >> 2) & 1) * 8 + 2 * (u & 3) + (u >> 3); }

// Bank spreading.  LDS rows narrower than 256 bytes (the 64 banks) start at
// only a few bank offsets, so 16 consecutive rows read at equal offsets would
// collide.  The 16-byte chunks of a row are XOR-permuted by the row's index
// among rows of equal bank offset: 16 consecutive rows then cover all banks.
template <int ROWB>
__device__ __forceinline__ int chunk_swz(int row) { return (row / (256 / ROWB)) & (ROWB / 16 - 1); }

// VBYTE: V^T rows start at unaligned addresses (N not a multiple of 4), so the
// V^T tiles are gathered byte by byte through registers instead of by 4-byte DMA.
template <int D, bool CAUSAL, bool OUT_BF16, bool VBYTE>
__global__ void __launch_bounds__(F8_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ VT,
               void* __restrict__ O, float* __restrict__ LSE, int BH, int G, int N, int nqt,
               float c /* scale * q_scale * k_scale * log2(e) */, float v_scale) {
    constexpr int BR = F8_BR, BC = F8_BC;
    constexpr int NKB = BC / 32;             // 32-key blocks per tile
    constexpr int NKS = D / 64;              // K-steps of S (64 dims each)
    constexpr int KCPR = D / 16;             // 16-byte chunks per K row
    constexpr int KTB = BC * D;              // K tile bytes
    constexpr int VTB = D * BC;              // V^T tile bytes (D rows of 64 keys)
    constexpr int KSPW = KTB / 1024 / 4;     // 1 KiB K segments per wave
    constexpr int KRPS = 1024 / D;           // K rows per segment
    constexpr int VSPW = VTB / 256 / 4;      // 256-byte V^T segments (4 rows) per wave
    static_assert(KSPW >= 1 && VSPW >= 1, "tile too small for four waves");

    __shared__ __attribute__((aligned(1024))) char kb0[KTB];
    __shared__ __attribute__((aligned(1024))) char kb1[KTB];
    __shared__ __attribute__((aligned(1024))) char vb0[VTB];
    __shared__ __attribute__((aligned(1024))) char vb1[VTB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt;
    fwd_tile_of(blockIdx.x, BH, G, nqt, CAUSAL, bh, qt);
    const int q0 = qt * BR;
    const size_t hoff = (size_t)bh * (size_t)N * D;            // bytes (and elements)
    const size_t kvoff = (size_t)(bh / G) * (size_t)N * D;
    const uint8_t* Kh = K + kvoff;
    const uint8_t* VTh = VT + kvoff;

    // Q^T fragments: lane (query, g) holds dims 64*ks + 32*g .. +31
    const int qrow = q0 + 32 * w + l32;
    i32x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (qrow < N) {
            const uint8_t* p = Q + hoff + (size_t)qrow * D + 64 * ks + 32 * g;
            lo = *reinterpret_cast<const uint4*>(p);
            hi = *reinterpret_cast<const uint4*>(p + 16);
        }
        qf[ks] = join8(lo, hi);
    }

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int nkt = (kv_end + BC - 1) / BC;
    const int wrow0 = q0 + 32 * w;
    const int nkt_w = (wrow0 >= N) ? 0 : (CAUSAL ? min(nkt, (wrow0 + 31) / BC + 1) : nkt);

    // K tile: row-major; V^T tile: D rows of 64 bytes in the key order
    // described above; both with their chunks permuted by chunk_swz.  Each tile is
    // addressed by buffer resources starting at the tile, so the per-lane
    // offsets below are fixed.  In a ragged last tile, K rows past N read as
    // zero (the resource ends with the head) and are masked; V^T keys past N
    // read the first keys of the next dim row (or zero after the last row),
    // finite values that meet P = 0.
    uint32_t k_dma[KSPW], v_dma[VSPW];
#pragma unroll
    for (int i = 0; i < KSPW; ++i) {
        const int row = (w * KSPW + i) * KRPS + lane / KCPR;
        const int slot = lane % KCPR;
        k_dma[i] = (uint32_t)(row * D + 16 * (slot ^ chunk_swz<D>(row)));
    }
#pragma unroll
    for (int i = 0; i < VSPW; ++i) {
        const int row = (w * VSPW + i) * 4 + lane / 16;            // dim
        const int u = ((lane % 16) ^ (chunk_swz<BC>(row) << 2));    // logical dword at this slot
        v_dma[i] = (uint32_t)((size_t)row * N + 4 * vt_src_dword(u));
    }
    // VBYTE: each thread gathers VBD dwords of the V^T tile (physical slot p
    // of dim row r), 4 keys each, byte by byte; keys past N are zero.
    constexpr int VBD = VBYTE ? D * 16 / F8_THREADS : 1;
    uint32_t vb_reg[VBD];
    auto vbyte_load = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < VBD; ++j) {
            const int i = tid + F8_THREADS * j;
            const int r = i / 16, p = i % 16;
            const int u = p ^ (chunk_swz<BC>(r) << 2);
            const int key0 = kt * BC + 4 * vt_src_dword(u);
            const uint8_t* src = VTh + (size_t)r * N + key0;
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (key0 + b < N) word |= (uint32_t)src[b] << (8 * b);
            vb_reg[j] = word;
        }
    };
    auto vbyte_store = [&](char* vdst) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < VBD; ++j) {
            const int i = tid + F8_THREADS * j;
            *reinterpret_cast<uint32_t*>(vdst + (i / 16) * BC + 4 * (i % 16)) = vb_reg[j];
        }
    };
    auto issue = [&](int kt, char* kdst, char* vdst) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh + (size_t)kt * BC * D, (uint32_t)(N - kt * BC) * D);
#pragma unroll
        for (int i = 0; i < KSPW; ++i) b2lds16(krs, k_dma[i], kdst + (w * KSPW + i) * 1024);
        if constexpr (VBYTE) {
            vbyte_load(kt);
        } else {
            const __amdgpu_buffer_rsrc_t vrs = make_rsrc(VTh + (size_t)kt * BC, (uint32_t)((size_t)D * N - kt * BC));
#pragma unroll
            for (int i = 0; i < VSPW; ++i) b2lds4(vrs, v_dma[i], vdst + (w * VSPW + i) * 256);
        }
    };

    // per-lane LDS offsets: K row l32 of block kb, chunks 4*ks + 2*g (+1)
    int k_off[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) k_off[ks][h] = l32 * D + 16 * ((4 * ks + 2 * g + h) ^ chunk_swz<D>(l32));
    //  V^T: dim row 32*mb + l32, logical chunks 2*g and 2*g + 1
    int v_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) v_off[h] = l32 * BC + 16 * ((2 * g + h) ^ chunk_swz<BC>(l32));

    const int last_visible = CAUSAL ? min(qrow, N - 1) : N - 1;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = zero16();
    float m_ref = -INFINITY;   // integer reference max, log2 units
    float l_run = 0.f;         // this lane's share of sum 2^8 p

    auto compute = [&](int kt, const char* Ks, const char* Vs) __attribute__((always_inline)) {
        // S^T = K Q^T
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const char* base = Ks + 32 * kb * D;
                const uint4 lo = *reinterpret_cast<const uint4*>(base + k_off[ks][0]);
                const uint4 hi = *reinterpret_cast<const uint4*>(base + k_off[ks][1]);
                s[kb] = mfma_f8(join8(lo, hi), qf[ks], s[kb]);
            }
        // mask; key kt*BC + 32*kb + 8*(r/4) + 4*g + r%4
        if ((kt * BC + BC > N) || (CAUSAL && kt * BC + BC - 1 > wrow0)) {
            const int lim = last_visible - kt * BC - 4 * g;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[kb][r];
        }
        // reference max: running max rounded up to an integer (log2 units)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float m_cand = ceilf(xor32_max(mx) * c);
        if (__any(m_cand > m_ref)) {
            const float m_new = fmaxf(m_ref, m_cand);
            const float alpha = exp2_fast(m_ref - m_new);   // a power of two; 0 while m_ref = -inf
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        }
        // e = 2^8 p = 2^(c s - m_ref + 8) <= 2^8; packed as e4m3 in key order
        // kb*16 + r (r = 4q + t), the B operand of O^T += V^T P^T
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        const float off = 8.f - m_use;
        i32x8 pb;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
                const float e0 = exp2_fast(fmaf(s[kb][4 * dw + 0], c, off));
                const float e1 = exp2_fast(fmaf(s[kb][4 * dw + 1], c, off));
                const float e2 = exp2_fast(fmaf(s[kb][4 * dw + 2], c, off));
                const float e3 = exp2_fast(fmaf(s[kb][4 * dw + 3], c, off));
                l_run += (e0 + e1) + (e2 + e3);
                pb[4 * kb + dw] = pack_fp8x4(e0, e1, e2, e3);
            }
        // O^T += V^T P^T
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
            const char* base = Vs + 32 * mb * BC;
            const uint4 lo = *reinterpret_cast<const uint4*>(base + v_off[0]);
            const uint4 hi = *reinterpret_cast<const uint4*>(base + v_off[1]);
            oacc[mb] = mfma_f8(join8(lo, hi), pb, oacc[mb]);
        }
    };
    auto step = [&](int kt, const char* Ks, const char* Vs, char* kn, char* vn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nkt) issue(kt + 1, kn, vn);
        if constexpr (VBYTE) {
            // the gathered V^T dwords of tile kt+1 go to LDS after this
            // tile's work; the next step's wait and barrier order them
            if (kt < nkt_w) compute(kt, Ks, Vs);
            if (kt + 1 < nkt) vbyte_store(vn);
        } else {
            if (kt < nkt_w) compute(kt, Ks, Vs);
        }
    };
    if (nkt > 0) {
        issue(0, kb0, vb0);
        if constexpr (VBYTE) vbyte_store(vb0);
    }
    for (int kt = 0; kt < nkt; kt += 2) {
        step(kt, kb0, vb0, kb1, vb1);
        if (kt + 1 < nkt) step(kt + 1, kb1, vb1, kb0, vb0);
    }

    const float l_tot = xor32_sum(l_run);   // sum of 2^8 p over the row
    if constexpr (OUT_BF16) {
        // bf16 O rows through the (now free) tile buffers, one per wave, so
        // each store writes whole rows (a direct store instruction would write
        // 16 bytes into each of 32 rows); chunks XOR-permuted by the row
        constexpr int ROWB = 2 * D, CH = D / 8;
        static_assert(32 * ROWB <= KTB && 32 * ROWB <= VTB, "a wave's O rows fit one tile buffer");
        const float inv = (l_tot > 0.f) ? v_scale / l_tot : 0.f;
        __syncthreads();                           // every wave is done with the tiles
        char* sb = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? vb0 : vb1;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int off = l32 * ROWB + 16 * ((4 * mb + rb) ^ (l32 % CH)) + 8 * g;
                *reinterpret_cast<uint2*>(sb + off) =
                    make_uint2(pack_bf16x2(oacc[mb][4 * rb + 0] * inv, oacc[mb][4 * rb + 1] * inv),
                               pack_bf16x2(oacc[mb][4 * rb + 2] * inv, oacc[mb][4 * rb + 3] * inv));
            }
        constexpr int RPP = 64 / CH;               // rows per pass, one chunk per lane
#pragma unroll
        for (int p = 0; p < 32 / RPP; ++p) {
            const int r = RPP * p + lane / CH, ch = lane % CH;
            const uint4 v4 = *reinterpret_cast<const uint4*>(sb + r * ROWB + 16 * (ch ^ (r % CH)));
            if (wrow0 + r < N)
                *reinterpret_cast<uint4*>(static_cast<__bf16*>(O) + (size_t)bh * N * D + (size_t)(wrow0 + r) * D +
                                          8 * ch) = v4;
        }
        if (qrow < N && g == 0)
            LSE[(size_t)bh * N + qrow] = (l_tot > 0.f) ? (m_ref - 8.f) * kLn2 + __logf(l_tot) : -INFINITY;
    } else if (qrow < N) {
        const float inv = (l_tot > 0.f) ? v_scale / l_tot : 0.f;
        const size_t orow = (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * mb + 8 * rb + 4 * g;
                const float o0 = oacc[mb][4 * rb + 0] * inv, o1 = oacc[mb][4 * rb + 1] * inv;
                const float o2 = oacc[mb][4 * rb + 2] * inv, o3 = oacc[mb][4 * rb + 3] * inv;
                if (OUT_BF16) {
                    *reinterpret_cast<uint2*>(static_cast<__bf16*>(O) + orow + d0) =
                        make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(O) + orow + d0) = make_float4(o0, o1, o2, o3);
                }
            }
        // LSE = ln(sum p) + m ln 2 = (m - 8) ln 2 + ln(sum 2^8 p)
        if (g == 0) LSE[(size_t)bh * N + qrow] = (l_tot > 0.f) ? (m_ref - 8.f) * kLn2 + __logf(l_tot) : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool OUT_BF16, bool VBYTE>
hipError_t launch(const Fp8FwdArgs& a) {
    const int BH = a.B * a.H;
    const int nqt = (a.N + F8_BR - 1) / F8_BR;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, OUT_BF16, VBYTE>), dim3((unsigned)(nqt * BH)), dim3(F8_THREADS), 0,
                       (hipStream_t)a.stream, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.vt, a.o,
                       a.lse, BH, a.H / a.Hkv, a.N, nqt, a.scale * a.q_scale * a.k_scale * kLog2e, a.v_scale);
    return hipGetLastError();
}

template <int D, bool VBYTE>
hipError_t dispatch_v(const Fp8FwdArgs& a) {
    if (a.out_bf16) return a.causal ? launch<D, true, true, VBYTE>(a) : launch<D, false, true, VBYTE>(a);
    return a.causal ? launch<D, true, false, VBYTE>(a) : launch<D, false, false, VBYTE>(a);
}

template <int D>
hipError_t dispatch(const Fp8FwdArgs& a) {
    return (a.N % 4 == 0) ? dispatch_v<D, false>(a) : dispatch_v<D, true>(a);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a) {
    if ((long long)((a.N + F8_BR - 1) / F8_BR) * a.B * a.H > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.d == 64 ? dispatch<64>(a) : dispatch<128>(a);
}

}  // namespace fa
