// Device helpers shared by the RMSNorm kernels (gfx950 / CDNA4, wave64).
//
// Layout conventions used by every row kernel:
//   * A row of H elements is handled by a "team" of TEAM lanes.  TEAM <= 64
//     keeps the team inside one wavefront (several rows per wavefront when
//     TEAM < 64); TEAM > 64 spans TEAM/64 wavefronts of one workgroup.
//   * Each lane owns NCH chunks of VEC consecutive elements; chunk c of lane l
//     starts at column (c * TEAM + l) * VEC, so a team's loads of one chunk
//     are contiguous (128-bit per lane when VEC * sizeof(T) == 16).
//   * Columns >= H are masked: they load as zero and are never stored, so
//     they add nothing to any sum (the mean still divides by H).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rms {

using bf16_t = uint16_t;  // storage of one bfloat16
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 128-bit access

constexpr int kWave = 64;

// 128-bit accesses.  NT = true marks a streaming access (each element is
// touched once): a nontemporal load/store that does not keep the line in the
// caches, which leaves them to the reused data (w, the dw partials).
template <bool NT>
__device__ __forceinline__ u32x4 ld128(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st128(void* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Element I/O: VEC elements of T <-> VEC floats.

template <typename T, int VEC>
struct Pack;  // raw storage of VEC elements

template <> struct Pack<float, 4> { u32x4 v; };
template <> struct Pack<float, 1> { float v; };
template <> struct Pack<bf16_t, 8> { u32x4 v; };
template <> struct Pack<bf16_t, 1> { bf16_t v; };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bfloat16 (nearest even) and pack, a in the low half.
// Converted as one two-element vector so that it compiles to gfx950's single
// two-operand v_cvt_pk_bf16_f32 (two scalar conversions compile to two of
// them, each with one operand, plus a shift and an or).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// The same rounding, one element at a time (two one-operand conversions, a
// shift and an or).  Kept for the residual backward's fp64 dx, where the
// single packed conversion led the compiler to chain every element's fp64
// arithmetic through one register pair (measured 86.0 -> 90.5 us for the
// bf16 16384 x 4096 row pass with dres); everywhere else the packed form is
// faster.
__device__ __forceinline__ uint32_t pack_bf16x2_split(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

__device__ __forceinline__ float round_to(float v, float*) { return v; }
__device__ __forceinline__ float round_to(float v, bf16_t*) {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v) << 16);
}

template <typename T, int VEC, bool NT = false>
__device__ __forceinline__ Pack<T, VEC> load_pack(const T* p) {
    Pack<T, VEC> r;
    if constexpr (VEC == 1) {
        if constexpr (NT) r.v = __builtin_nontemporal_load(p);
        else r.v = *p;
    } else {
        r.v = ld128<NT>(p);
    }
    return r;
}

template <typename T, int VEC>
__device__ __forceinline__ Pack<T, VEC> zero_pack() {
    Pack<T, VEC> r;
    if constexpr (VEC == 1) {
        r.v = 0;
    } else {
        r.v = u32x4{0u, 0u, 0u, 0u};
    }
    return r;
}

// Makes p's value opaque to the optimiser (an empty asm that may "change"
// it), so that values derived from p are recomputed after this point rather
// than kept live from before it, and nothing derived from p is hoisted out of
// a loop that calls this.
template <typename T, int VEC>
__device__ __forceinline__ void opaque(Pack<T, VEC>& p) {
    asm volatile("" : "+v"(p.v));
}

template <typename T, int VEC>
__device__ __forceinline__ void unpack(const Pack<T, VEC>& p, float (&f)[VEC]) {
    if constexpr (sizeof(T) == 4 && VEC == 4) {
        f[0] = __uint_as_float(p.v.x); f[1] = __uint_as_float(p.v.y);
        f[2] = __uint_as_float(p.v.z); f[3] = __uint_as_float(p.v.w);
    } else if constexpr (sizeof(T) == 4 && VEC == 1) {
        f[0] = p.v;
    } else if constexpr (VEC == 8) {
        f[0] = bf16_lo(p.v.x); f[1] = bf16_hi(p.v.x);
        f[2] = bf16_lo(p.v.y); f[3] = bf16_hi(p.v.y);
        f[4] = bf16_lo(p.v.z); f[5] = bf16_hi(p.v.z);
        f[6] = bf16_lo(p.v.w); f[7] = bf16_hi(p.v.w);
    } else {
        f[0] = __uint_as_float((uint32_t)p.v << 16);
    }
}

template <typename T, int VEC, bool NT = false>
__device__ __forceinline__ void store_vec(T* p, const float (&f)[VEC]) {
    if constexpr (sizeof(T) == 4 && VEC == 4) {
        st128<NT>(p, u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                       __float_as_uint(f[3])});
    } else if constexpr (sizeof(T) == 4 && VEC == 1) {
        if constexpr (NT) __builtin_nontemporal_store(f[0], reinterpret_cast<float*>(p));
        else *reinterpret_cast<float*>(p) = f[0];
    } else if constexpr (VEC == 8) {
        st128<NT>(p, u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7])});
    } else {
        const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)f[0]);
        if constexpr (NT) __builtin_nontemporal_store(b, p);
        else *p = b;
    }
}

// ---------------------------------------------------------------------------
// Raw buffer access.  A buffer resource holds a base address and a size in
// bytes; a load at an offset at or past the size returns zero without
// reading memory, and a store there is dropped.  Row kernels address a block
// of rows through resources sized to the rows that exist, and give lanes of
// columns past H an offset past every size (kBufOutside), so neither needs a
// branch, a mask or a substitute address.
constexpr int kBufWord3 = 0x00020000;          // untyped access, 32-bit data format
constexpr uint32_t kBufOutside = 0x80000000u;  // beyond any resource made here
// Cache-policy bits of the aux operand (gfx940-family encoding).
constexpr int kAuxNt = 2;
constexpr int kAuxSc1 = 16;

typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufWord3);
}

template <typename T, int VEC, bool NT = false>
__device__ __forceinline__ Pack<T, VEC> buf_load_pack(BufRes r, uint32_t off) {
    constexpr int aux = NT ? kAuxNt : 0;
    Pack<T, VEC> p;
    if constexpr (VEC == 1 && sizeof(T) == 2) {
        p.v = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, aux);
    } else if constexpr (VEC == 1) {
        p.v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, aux));
    } else {
        p.v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, aux);
    }
    return p;
}

// 16 bytes per lane from a resource straight into LDS: lane l's bytes land
// at wave_base + 16 l (wave_base: the wavefront's own LDS region, the same
// address in every lane).  Completion is counted by vmcnt like any load; the
// compiler does not order a later LDS read after it, so callers wait
// explicitly.  The body exists in the device pass only (an LDS address space
// has no meaning in the host pass, whose kernel stubs it would otherwise
// drop).
template <int AUX>
__device__ __forceinline__ void buf_load_lds16(BufRes r, void* wave_base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)wave_base,
                                             16, (int)off, 0, 0, AUX);
#else
    (void)r;
    (void)wave_base;
    (void)off;
#endif
}

__device__ __forceinline__ float buf_load_f32(BufRes r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// store_vec through a resource.  Streaming (NT) stores are nontemporal with
// device scope (nt sc1), so the line is written through the XCD's L2 rather
// than left dirty there for the write-back at the end of the kernel
// (measured on the bf16 4096 x 4096 forward + backward step: 35.2-35.5 ->
// 34.9-35.0 us against nontemporal stores alone).
template <typename T, int VEC, bool NT = false, bool kSplitCvt = false>
__device__ __forceinline__ void buf_store_vec(BufRes r, uint32_t off, const float (&f)[VEC]) {
    constexpr int aux = NT ? (kAuxNt | kAuxSc1) : 0;
    if constexpr (sizeof(T) == 4 && VEC == 4) {
        const u32x4 v{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, aux);
    } else if constexpr (sizeof(T) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f[0]), r, (int)off, 0, aux);
    } else if constexpr (VEC == 8 && kSplitCvt) {
        const u32x4 v{pack_bf16x2_split(f[0], f[1]), pack_bf16x2_split(f[2], f[3]),
                      pack_bf16x2_split(f[4], f[5]), pack_bf16x2_split(f[6], f[7])};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, aux);
    } else if constexpr (VEC == 8) {
        const u32x4 v{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7])};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, aux);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)f[0]), r,
                                              (int)off, 0, aux);
    }
}

// Products for the per-row fp64 sums.  Squares are formed in fp64 (the
// caller's add contracts with the multiply into one fp64 fused multiply-add):
// exact for every fp32 or bf16 value, and free of the overflow (|x| beyond
// about 2^64) and underflow (|x| below about 2^-63) of an fp32 square.  For
// bf16 inputs w*dy*x is formed in fp32, where it is exact (8-bit significands:
// 24 bits in all) while |w dy x| lies between 2^-126 and 2^128, the range
// include/rmsnorm.h states; for fp32 inputs it is formed in fp64.  (Forming
// it in fp64 for bf16 as well raised the register use of the row-in-LDS
// backward until it spilled.)
__device__ __forceinline__ double sq64(float v, float*) { return (double)v * (double)v; }
__device__ __forceinline__ double sq64(float v, bf16_t*) { return (double)v * (double)v; }
__device__ __forceinline__ double prod2_64(float a, float b, float*) {
    return (double)a * (double)b;
}
__device__ __forceinline__ double prod2_64(float a, float b, bf16_t*) { return (double)(a * b); }
__device__ __forceinline__ double prod3_64(float a, float b, float c, float*) {
    return (double)a * (double)b * (double)c;
}
__device__ __forceinline__ double prod3_64(float a, float b, float c, bf16_t*) {
    return (double)((a * b) * c);
}

// r = 1/sqrt(m) in fp64 for m >= 0: the hardware reciprocal square root
// refined by one Newton step r' = r (3 - m r^2) / 2, which squares its
// relative error, leaving r within a few fp64 ulps (so its fp32 rounding is
// the correctly rounded fp32 of the exact value except on exact ties).  About
// a fifth of the instructions of 1.0 / sqrt(m).  m = 0 returns +inf and
// m = +inf returns 0 (the hardware value; the Newton step would give NaN).
__device__ __forceinline__ double rsqrt_f64(double m) {
    const double r = __builtin_amdgcn_rsq(m);
    return (m > 0.0 && m < __builtin_inf()) ? r * (1.5 - 0.5 * m * (r * r)) : r;
}

// ---------------------------------------------------------------------------
// Team all-reductions.  Every lane of a team ends with the bitwise-identical
// sum (each step adds a value to its partner's, a + b == b + a exactly).
// All 64 lanes of the wavefront must be active.

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16 lanes

// Every control above gives each lane a source lane inside its own 16-lane
// row, and all rows and banks are enabled, so every lane is written from its
// source and the instruction's "old" operand is never read: mov_dpp leaves it
// unspecified, which spares the two zero moves per 64-bit step that an
// explicit old value costs.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    int2 p = __builtin_bit_cast(int2, v);
    p.x = __builtin_amdgcn_mov_dpp(p.x, CTRL, 0xF, 0xF, false);
    p.y = __builtin_amdgcn_mov_dpp(p.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, p);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    int2 p = __builtin_bit_cast(int2, v);
    p.x = __builtin_amdgcn_readlane(p.x, lane);
    p.y = __builtin_amdgcn_readlane(p.y, lane);
    return __builtin_bit_cast(double, p);
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over aligned groups of TEAM lanes (TEAM in 1..64, a power of two).
template <int TEAM, typename V>
__device__ __forceinline__ V team_sum_wave(V v) {
    static_assert(TEAM >= 1 && TEAM <= 64 && (TEAM & (TEAM - 1)) == 0, "TEAM");
    auto step = [](V a, auto ctrl_tag) {
        constexpr int C = decltype(ctrl_tag)::value;
        if constexpr (sizeof(V) == 8) return a + dpp_f64<C>(a);
        else return a + dpp_f32<C>(a);
    };
    if constexpr (TEAM >= 2) v = step(v, std::integral_constant<int, kQuadXor1>{});
    if constexpr (TEAM >= 4) v = step(v, std::integral_constant<int, kQuadXor2>{});
    if constexpr (TEAM >= 8) v = step(v, std::integral_constant<int, kRowHalfMirror>{});
    if constexpr (TEAM >= 16) v = step(v, std::integral_constant<int, kRowMirror>{});
    if constexpr (TEAM >= 32) {
        // Rows of 16 lanes now hold their sums; combine rows through
        // lane reads (uniform values) in a fixed order.
        V s0, s1, s2, s3;
        if constexpr (sizeof(V) == 8) {
            s0 = readlane_f64(v, 0); s1 = readlane_f64(v, 16);
            s2 = readlane_f64(v, 32); s3 = readlane_f64(v, 48);
        } else {
            s0 = readlane_f32(v, 0); s1 = readlane_f32(v, 16);
            s2 = readlane_f32(v, 32); s3 = readlane_f32(v, 48);
        }
        if constexpr (TEAM == 64) {
            v = (s0 + s1) + (s2 + s3);
        } else {
            const bool upper = (threadIdx.x & 32) != 0;
            v = upper ? (s2 + s3) : (s0 + s1);
        }
    }
    return v;
}

// Sum over a team of TEAM lanes; TEAM > 64 spans TEAM/64 wavefronts and uses
// `lds` (at least TEAM/64 values per team).  Contains __syncthreads() when
// TEAM > 64, so every thread of the workgroup must call it.
template <int TEAM, typename V>
__device__ __forceinline__ V team_sum(V v, V* lds) {
    if constexpr (TEAM <= 64) {
        return team_sum_wave<TEAM>(v);
    } else {
        constexpr int NW = TEAM / kWave;
        v = team_sum_wave<64>(v);
        const int lt = threadIdx.x % TEAM;
        const int team = threadIdx.x / TEAM;
        V* slot = lds + team * NW;
        if ((lt & (kWave - 1)) == 0) slot[lt / kWave] = v;
        __syncthreads();
        V s = slot[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) s += slot[k];
        __syncthreads();  // slots may be reused by the next reduction
        return s;
    }
}

// As team_sum, with one barrier instead of two: the caller alternates
// between two disjoint slot sets `lds` on successive calls, so a set is only
// rewritten after every thread has passed the barrier of the call in between
// (which follows its reads of that set).  Contains __syncthreads() when
// TEAM > 64.
template <int TEAM, typename V>
__device__ __forceinline__ V team_sum_alt(V v, V* lds) {
    if constexpr (TEAM <= 64) {
        return team_sum_wave<TEAM>(v);
    } else {
        constexpr int NW = TEAM / kWave;
        v = team_sum_wave<64>(v);
        const int lt = threadIdx.x % TEAM;
        const int team = threadIdx.x / TEAM;
        V* slot = lds + team * NW;
        if ((lt & (kWave - 1)) == 0) slot[lt / kWave] = v;
        __syncthreads();
        V s = slot[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) s += slot[k];
        return s;
    }
}

}  // namespace rms
