// Plain streams for the benchmark's ceiling figures (not part of the RMSNorm
// library): the fastest access shapes measured for moving the row tensors'
// bytes on gfx950 and nothing else.  Each 512-lane workgroup moves one 8 KB
// block of every stream: NR streams read with 128-bit nontemporal loads,
// summed lane-wise so that every load is used, and NW streams written with
// 128-bit nontemporal stores.  No reduction, no weights, no second pass: the
// time a kernel needs just to read and write the same bytes.  Two access
// kinds, which lead on different patterns by 1-2%: plain global accesses
// (KIND 0), and buffer-resource accesses with device-scope stores (KIND 1:
// nt loads, nt sc1 stores, as the library's row kernels issue them).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kLanes = 512;
constexpr int64_t kBlockBytes = kLanes * 16;

typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr int kAuxNt = 2, kAuxSc1 = 16;  // cache-policy bits (gfx940-family encoding)

// A resource over one workgroup's 8 KB block of a stream.
__device__ __forceinline__ BufRes block_rsrc(const u32x4* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(p) + (int64_t)blockIdx.x * kLanes,
                                             (short)0, (int)kBlockBytes, 0x00020000);
}

template <int NR, int NW, int KIND>
__global__ __launch_bounds__(kLanes) void stream_kernel(const u32x4* __restrict__ a,
                                                        const u32x4* __restrict__ b,
                                                        const u32x4* __restrict__ c,
                                                        u32x4* __restrict__ d,
                                                        u32x4* __restrict__ e) {
    if constexpr (KIND == 0) {
        const int64_t i = (int64_t)blockIdx.x * kLanes + threadIdx.x;
        u32x4 v = __builtin_nontemporal_load(a + i);
        if constexpr (NR > 1) v += __builtin_nontemporal_load(b + i);
        if constexpr (NR > 2) v += __builtin_nontemporal_load(c + i);
        __builtin_nontemporal_store(v, d + i);
        if constexpr (NW > 1) __builtin_nontemporal_store(v + 1u, e + i);
    } else {
        const int off = (int)threadIdx.x * 16;
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(block_rsrc(a), off, 0, kAuxNt);
        if constexpr (NR > 1)
            v += __builtin_amdgcn_raw_buffer_load_b128(block_rsrc(b), off, 0, kAuxNt);
        if constexpr (NR > 2)
            v += __builtin_amdgcn_raw_buffer_load_b128(block_rsrc(c), off, 0, kAuxNt);
        __builtin_amdgcn_raw_buffer_store_b128(v, block_rsrc(d), off, 0, kAuxNt | kAuxSc1);
        if constexpr (NW > 1)
            __builtin_amdgcn_raw_buffer_store_b128(v + 1u, block_rsrc(e), off, 0, kAuxNt | kAuxSc1);
    }
}

template <int NR, int NW>
hipError_t launch(int kind, const void* a, const void* b, const void* c, void* d, void* e,
                  int64_t blocks, hipStream_t s) {
    if (kind == 0) {
        hipLaunchKernelGGL((stream_kernel<NR, NW, 0>), dim3((unsigned)blocks), dim3(kLanes), 0, s,
                           (const u32x4*)a, (const u32x4*)b, (const u32x4*)c, (u32x4*)d, (u32x4*)e);
    } else {
        hipLaunchKernelGGL((stream_kernel<NR, NW, 1>), dim3((unsigned)blocks), dim3(kLanes), 0, s,
                           (const u32x4*)a, (const u32x4*)b, (const u32x4*)c, (u32x4*)d, (u32x4*)e);
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Reads streams a (, b, c) and writes d (, e), `bytes` each, on `stream`,
// with access kind `kind` (0 or 1, above).  nr in 1..3 and nw in 1..2; every
// pointer the pattern uses non-null and 16-byte aligned; bytes a positive
// multiple of 8192 (whole workgroup blocks), at most 2^31 - 1 blocks.
// Returns 0, 1 for arguments outside these limits (nothing launched), 2 for
// a launch error.
int bench_stream(int nr, int nw, int kind, const void* a, const void* b, const void* c, void* d,
                 void* e, int64_t bytes, hipStream_t stream) {
    if (nr < 1 || nr > 3 || nw < 1 || nw > 2 || kind < 0 || kind > 1) return 1;
    if (bytes <= 0 || bytes % kBlockBytes != 0 || bytes / kBlockBytes > INT32_MAX) return 1;
    const void* in[3] = {a, b, c};
    void* out[2] = {d, e};
    for (int k = 0; k < nr; ++k)
        if (!in[k] || (uintptr_t)in[k] % 16 != 0) return 1;
    for (int k = 0; k < nw; ++k)
        if (!out[k] || (uintptr_t)out[k] % 16 != 0) return 1;
    const int64_t blocks = bytes / kBlockBytes;
    hipError_t err;
    switch (nr * 10 + nw) {
        case 11: err = launch<1, 1>(kind, a, b, c, d, e, blocks, stream); break;
        case 12: err = launch<1, 2>(kind, a, b, c, d, e, blocks, stream); break;
        case 21: err = launch<2, 1>(kind, a, b, c, d, e, blocks, stream); break;
        case 22: err = launch<2, 2>(kind, a, b, c, d, e, blocks, stream); break;
        case 31: err = launch<3, 1>(kind, a, b, c, d, e, blocks, stream); break;
        default: err = launch<3, 2>(kind, a, b, c, d, e, blocks, stream); break;
    }
    return err == hipSuccess ? 0 : 2;
}

}  // extern "C"
