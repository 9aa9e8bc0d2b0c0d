// fa_internal.hpp -- host-side launch interface between the C ABI layer and
// the kernel translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Hkv, N, d;   // H query heads; Hkv K/V heads, dividing H
    bool in_bf16;    // false: fp32 inputs
    bool out_bf16;   // O element type
    bool causal;
    float scale;
    void* stream;
};

// fp8 (e4m3) forward: Q [B,H,N,d], K [B,Hkv,N,d], V transposed [B,Hkv,d,N];
// real value = stored value * the tensor's scale
struct Fp8FwdArgs {
    const void* q;
    const void* k;
    const void* vt;
    float q_scale, k_scale, v_scale;
    void* o;
    float* lse;
    int B, H, Hkv, N, d;
    bool out_bf16;
    bool causal;
    float scale;
    void* stream;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;    // workspace: [B,H,N] fp32, rowsum(dO * O) (written by the dQ kernel)
    float* lse2;     // workspace: [B,H,N] fp32, LSE log2 e (written by the dQ kernel)
    float* pdk;      // workspace when split: [B*H/s, N, d] fp32 partial dK^T rows per head group
    float* pdv;      // workspace when split: [B*H/s, N, d] fp32 partial dV^T rows per head group
    int split;       // bwd_split_heads(B, H, Hkv, N): query heads per split workgroup, 0 = no split
    int B, H, Hkv, N, d;
    bool o_bf16;
    bool causal;
    float scale;
    void* stream;
};

// Paged KV cache: pool [num_pages, Hkv, page_size, d]; sequence b owns pages
// block_table[b * max_pages + 0 ..] in token order and has seq_lens[b] tokens.
struct Paging {
    const int* block_table;   // null: contiguous cache
    const int* seq_lens;
    int num_pages;
    int max_pages;
    int ps_log2;              // page_size = 1 << ps_log2 (>= 32)
    int Hkv;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;      // may be null
    float* o_part;   // workspace: [B,H,S,d] fp32
    float* lse_part; // workspace: [B,H,S] fp32
    int B, H, Hkv, L, d;
    int splits;      // S >= 1; contiguous: every split non-empty
    int chunk;       // keys per split, a multiple of 32
    float scale;
    void* stream;
    Paging paging;   // block_table == nullptr for a contiguous cache (L = its length);
                     // paged: L = max_pages * page_size
};

// Backward with grouped heads: the dK/dV kernel normally sums the G query
// heads of a K/V head inside one workgroup (one per K/V head and 128-key
// tile).  When that grid is small -- below two workgroups per CU -- the
// uneven causal work of the key tiles decides the run time, so the query heads
// are split into groups of s, each with workgroups of its own, writing fp32
// partial dK/dV that a second kernel sums over the groups in a fixed order.
// s is chosen to give just enough workgroups: measured on MI355X with 4 query
// heads per K/V head, a split into single heads gains 13% at 256 workgroups
// and loses 18-29% at 512, where the partials' extra traffic outweighs the
// better balance.
constexpr int kBwdKeyTile = 128;
constexpr long long kBwdSplitBelow = 512;
// Returns s, the query heads one dK/dV workgroup visits on the split path:
// the largest divisor of G = H/Hkv below G that still gives at least
// kBwdSplitBelow workgroups (1 if none does); 0 when the (K/V head, key tile)
// pairs alone are enough and no split is taken.
inline int bwd_split_heads(int B, int H, int Hkv, int N) {
    if (Hkv >= H) return 0;
    const long long nkt = (N + kBwdKeyTile - 1) / kBwdKeyTile;
    const long long pairs = nkt * B * Hkv;
    if (pairs >= kBwdSplitBelow) return 0;
    const int G = H / Hkv;
    for (int s = G / 2; s > 1; --s)
        if (G % s == 0 && pairs * (G / s) >= kBwdSplitBelow) return s;
    return 1;
}

// Decode kernels by group size G = H/Hkv:
//  - G = 2 and 3, and G = 4 over at least 64 (batch, cache head) pairs: the
//    small-group kernel (the per-head kernel's streaming layout with the
//    group's heads on the same lanes).  Measured on MI355X at L = 8192 it
//    streams 6.3-6.9 TB/s from batch 16 up, against 5.5-6.0 for the MFMA
//    grouped kernel; with G = 4 at batch 1-4 and 8 cache heads the MFMA
//    kernel's shorter chunks were 1-11% faster.
//  - other G in [2, 32]: the MFMA grouped kernel;
//  - G = 1 or G > 32: the per-query-head kernel.
constexpr int kDecodeMaxGroup = 32;
inline int decode_small_group(int B, int H, int Hkv) {
    const int G = H / Hkv;
    if (G == 2 || G == 3) return G;
    if (G == 4 && (long long)B * Hkv >= 64) return 4;
    return 0;
}
inline bool decode_group_path(int B, int H, int Hkv) {
    const int G = H / Hkv;
    return G >= 2 && G <= kDecodeMaxGroup && decode_small_group(B, H, Hkv) == 0;
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

// Device address of the static scratch array (FA_NOALLOC_SCRATCH_BYTES) on
// the current device; looked up once per device.
hipError_t decode_scratch(void** ptr);

}  // namespace fa
