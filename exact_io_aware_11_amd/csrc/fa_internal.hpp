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
    float* delta;    // workspace: [B,H,N] fp32, rowsum(dO * O)
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

// Decode takes the grouped-query kernel (each cache head read once for all
// the query heads sharing it) when 2 <= H/Hkv <= kDecodeMaxGroup; otherwise
// the per-query-head kernel.
constexpr int kDecodeMaxGroup = 32;
inline bool decode_group_path(int H, int Hkv) {
    const int G = H / Hkv;
    return G >= 2 && G <= kDecodeMaxGroup;
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

}  // namespace fa
