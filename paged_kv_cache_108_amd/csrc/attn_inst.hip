// Instantiations of the attention kernels for one cache type and head dim,
// chosen at compile time (-DPKV_INST_KV=0|1|2 for f32|bf16|fp8 caches,
// -DPKV_INST_D=64|128); the build compiles this file once per pair, in
// parallel. pick_kernel returns the kernel for a block size and mode;
// pick_plan_kernel the planned kernel and pick_gather_kernel the gather-only
// kernel for a block size.
#include "attn_kernels.h"

#ifndef PKV_INST_KV
#error "PKV_INST_KV must be defined (0: f32, 1: bf16, 2: fp8)"
#endif
#ifndef PKV_INST_D
#error "PKV_INST_D must be defined (64 or 128)"
#endif

namespace pkv_dev {

namespace {

template <int KV, int D, int MODE, int NT, bool CACHED = false>
AttnKernel stream_for_bs(int bs) {
    switch (bs) {
        case 8: return paged_attn_stream_kernel<KV, D, 8, MODE, NT, CACHED>;
        case 16: return paged_attn_stream_kernel<KV, D, 16, MODE, NT, CACHED>;
        case 32: return paged_attn_stream_kernel<KV, D, 32, MODE, NT, CACHED>;
        case 64: return paged_attn_stream_kernel<KV, D, 64, MODE, NT, CACHED>;
        case 128: return paged_attn_stream_kernel<KV, D, 128, MODE, NT, CACHED>;
    }
    return nullptr;
}

template <int KV, int D>
AttnKernel partition_for_bs(int bs) {
    switch (bs) {
        case 8: return paged_attn_partition_kernel<KV, D, 8>;
        case 16: return paged_attn_partition_kernel<KV, D, 16>;
        case 32: return paged_attn_partition_kernel<KV, D, 32>;
        case 64: return paged_attn_partition_kernel<KV, D, 64>;
        case 128: return paged_attn_partition_kernel<KV, D, 128>;
    }
    return nullptr;
}

}  // namespace

// tiles: 16-column MFMA tiles per pass (query windows: 1 or wide_tiles(D));
// cached: plain K/V loads (wide windows of several passes)
template <int KV, int D>
AttnKernel pick_kernel(int bs, int mode, int tiles, bool partition, bool cached) {
    if (partition) return partition_for_bs<KV, D>(bs);
    switch (mode) {
        case SM_WINDOW:
            if (tiles == 1) return stream_for_bs<KV, D, SM_WINDOW, 1>(bs);
            return cached ? stream_for_bs<KV, D, SM_WINDOW, wide_tiles(D), true>(bs)
                          : stream_for_bs<KV, D, SM_WINDOW, wide_tiles(D)>(bs);
        case SM_STEP: return stream_for_bs<KV, D, SM_STEP, 1>(bs);
        case SM_SHARED: return stream_for_bs<KV, D, SM_SHARED, 1>(bs);
        default: return stream_for_bs<KV, D, SM_DECODE, 1>(bs);
    }
}

template AttnKernel pick_kernel<PKV_INST_KV, PKV_INST_D>(int, int, int, bool, bool);

template <int KV, int D, int PM, bool CACHED>
AttnKernel plan_for_bs(int bs) {
    switch (bs) {
        case 8: return paged_attn_plan_kernel<KV, D, 8, PM, CACHED>;
        case 16: return paged_attn_plan_kernel<KV, D, 16, PM, CACHED>;
        case 32: return paged_attn_plan_kernel<KV, D, 32, PM, CACHED>;
        case 64: return paged_attn_plan_kernel<KV, D, 64, PM, CACHED>;
        case 128: return paged_attn_plan_kernel<KV, D, 128, PM, CACHED>;
    }
    return nullptr;
}

// mode: PM_ATTN, PM_STEP, PM_WINDOW or PM_WINDOW2 (two tiles); cached:
// cacheable K/V loads (decode modes, for plans that list shared blocks; two-
// tile windows of several query groups, whose groups read the same blocks)
template <int KV, int D>
AttnKernel pick_plan_kernel(int bs, int mode, bool cached) {
    switch (mode) {
        case PM_ATTN: return cached ? plan_for_bs<KV, D, PM_ATTN, true>(bs) : plan_for_bs<KV, D, PM_ATTN, false>(bs);
        case PM_STEP: return cached ? plan_for_bs<KV, D, PM_STEP, true>(bs) : plan_for_bs<KV, D, PM_STEP, false>(bs);
        case PM_WINDOW: return cached ? nullptr : plan_for_bs<KV, D, PM_WINDOW, false>(bs);
        case PM_WINDOW2:
            return cached ? plan_for_bs<KV, D, PM_WINDOW2, true>(bs) : plan_for_bs<KV, D, PM_WINDOW2, false>(bs);
    }
    return nullptr;
}

template AttnKernel pick_plan_kernel<PKV_INST_KV, PKV_INST_D>(int, int, bool);

template <int KV, int D, bool CACHED>
AttnKernel gather_for_bs(int bs) {
    switch (bs) {
        case 8: return paged_gather_kernel<KV, D, 8, CACHED>;
        case 16: return paged_gather_kernel<KV, D, 16, CACHED>;
        case 32: return paged_gather_kernel<KV, D, 32, CACHED>;
        case 64: return paged_gather_kernel<KV, D, 64, CACHED>;
        case 128: return paged_gather_kernel<KV, D, 128, CACHED>;
    }
    return nullptr;
}

// cached: the loads of a plan marked for shared blocks, as the planned kernel
template <int KV, int D>
AttnKernel pick_gather_kernel(int bs, bool cached) {
    return cached ? gather_for_bs<KV, D, true>(bs) : gather_for_bs<KV, D, false>(bs);
}

template AttnKernel pick_gather_kernel<PKV_INST_KV, PKV_INST_D>(int, bool);

}  // namespace pkv_dev
