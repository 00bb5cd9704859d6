// ss_tiles.h -- global -> LDS staging of time chunks for the scan kernels.
//
// A chunk is a set of tiles, each 16 rows x KT time steps of one tensor
// (rows are channels for u / delta / z / dout and state indices for B / C).
// Every thread owns a fixed set of 16-byte slots of those tiles.  Source
// pointers and LDS offsets of the slots are computed once.  A full chunk is
// then staged with one unguarded 16-byte global load per slot, kept as raw
// words in registers until the chunk before it is done (so the loads stay in
// flight across a whole chunk of compute), and only the ragged last chunk
// takes the guarded element path.  Tiles span whole wavefronts of slots, so
// the tile a slot belongs to is uniform across a wavefront.
#pragma once

#include "ss_device.h"

namespace ssk {

struct alignas(16) Raw16 {
    uint32_t w[4];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads / stores through explicit global-address-space pointers, so
// the compiler issues global (not flat) memory instructions.
__device__ __forceinline__ u32x4 ld_global16(const void *p) {
    return *(const __attribute__((address_space(1))) u32x4 *)(p);
}
__device__ __forceinline__ void st_global16(void *p, u32x4 v) {
    *(__attribute__((address_space(1))) u32x4 *)(p) = v;
}
// Single-element global load.  Generic (flat) loads would make every later
// wait on the vector-memory counter a full drain, since a pending flat
// access may be an LDS access too.
template <typename T>
__device__ __forceinline__ T ld_global(const T *p) {
    return *(const __attribute__((address_space(1))) T *)(p);
}
template <typename T>
__device__ __forceinline__ void st_global(T *p, T v) {
    *(__attribute__((address_space(1))) T *)(p) = v;
}

// Four consecutive elements of T (16 bytes of f32, 8 of bf16) widened to
// f32, and the reverse; the address must be aligned to the access size.
template <typename T>
__device__ __forceinline__ void ld4(const T *p, float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        const u32x4 r = ld_global16(p);
        v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 r = *(const __attribute__((address_space(1))) u32x2 *)(p);
        const uint32_t r0 = r.x, r1 = r.y;
        v[0] = __uint_as_float(r0 << 16); v[1] = __uint_as_float(r0 & 0xffff0000u);
        v[2] = __uint_as_float(r1 << 16); v[3] = __uint_as_float(r1 & 0xffff0000u);
    }
}
template <typename T>
__device__ __forceinline__ void st4(T *p, const float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        u32x4 r;
        r.x = __float_as_uint(v[0]); r.y = __float_as_uint(v[1]);
        r.z = __float_as_uint(v[2]); r.w = __float_as_uint(v[3]);
        st_global16(p, r);
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        u32x2 r;
        r.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
        r.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
        *(__attribute__((address_space(1))) u32x2 *)(p) = r;
    }
}

// Address = base + a 32-bit byte offset.  With a base that is uniform
// across the wavefront (scalar registers), the compiler uses the scalar-base
// form of the global instructions and needs no 64-bit vector address math.
template <typename T>
__device__ __forceinline__ const T *at_bytes(const T *base, uint32_t off) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}
template <typename T>
__device__ __forceinline__ T *at_bytes(T *base, uint32_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + off);
}

// Element tensors (u, delta, z, dout) reach the lanes that own their
// elements straight from global memory when 4 bytes wide; 2-byte elements
// are staged through LDS with the B / C tiles (per-lane 2-byte loads split
// every cache line into four requests, which costs more than the LDS round
// trip).
template <typename T>
constexpr bool kStageElems = sizeof(T) == 2;

// One tile of a chunk.
template <typename T>
struct TileSrc {
    const T *base;     // element (row 0, t = 0) of the tile; nullptr = absent (zeros)
    int64_t row_stride;
    int valid_rows;    // rows >= valid_rows read as zeros
    uint32_t lds_off;  // byte offset of the tile in the kernel's LDS buffer
    int pitch;         // LDS row pitch in elements of the LDS type
    bool to_f32;       // stash as f32 (else as T)
};

template <typename T, int VEC, int KT, int NTILES, int NTHREADS>
struct ChunkStager {
    static_assert(VEC * sizeof(T) == 16 || VEC == 1, "slots are 16 bytes or single elements");
    static constexpr int kVecPerRow = KT / VEC;
    static constexpr int kVecPerTile = 16 * kVecPerRow;
    static constexpr int kSlots = (NTILES * kVecPerTile + NTHREADS - 1) / NTHREADS;
    static constexpr int kWords = (VEC * sizeof(T) + 3) / 4;
    // tiles of whole wavefronts of slots keep the tile index (and so its
    // descriptor) uniform across a wavefront
    static constexpr bool kUniformTile = kVecPerTile % 64 == 0;
    static_assert(kSlots <= 32, "slot flags fit one 32-bit mask");

    // Per slot: the tile's base (uniform across the wavefront when
    // kUniformTile, so in scalar registers) and 32-bit per-lane offsets.
    // A slot of an absent tile or of a row past the last valid one is not
    // live: it still loads (from row 0 of tile 0 or of its own tile, which
    // always exist, so a full chunk's loads need no branch) but its words are
    // garbage; the ragged chunk reads zeros for it.  Kernels never read an
    // absent tile and give rows past the last valid one no part in any sum
    // across rows.
    const T *base[kSlots];  // element (row 0, t = 0) of the tile the slot loads from
    uint32_t goff[kSlots];  // the lane's element offset in that tile (row * stride + col)
    uint32_t dst[kSlots];   // LDS byte offset
    bool f32[kSlots];       // stash as f32 (else as T); uniform
    bool used[kSlots];      // slot maps to a tile; uniform
    uint32_t live = 0;      // bit k: slot k's words are real data
    uint32_t reg[kSlots][kWords];

    __device__ static int slot_col(int tid, int k) {
        return ((tid + k * NTHREADS) % kVecPerRow) * VEC;
    }

    // `desc(i)` returns the TileSrc of tile i (called with constant i only);
    // tile 0 must be present.
    template <typename Desc>
    __device__ __forceinline__ void init(Desc desc, int tid) {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const int slot = tid + k * NTHREADS;
            const int tile = kUniformTile ? __builtin_amdgcn_readfirstlane(slot / kVecPerTile)
                                          : slot / kVecPerTile;
            const int rem = slot % kVecPerTile;
            const int row = rem / kVecPerRow;
            const int col = (rem % kVecPerRow) * VEC;
            base[k] = desc(0).base;
            goff[k] = uint32_t(col);
            dst[k] = 0;
            f32[k] = false;
            used[k] = tile < NTILES;
            if (tile < NTILES) {
                TileSrc<T> ts = desc(0);
#pragma unroll
                for (int i = 1; i < NTILES; i++)
                    if (tile == i) ts = desc(i);
                if (ts.base && row < ts.valid_rows) live |= 1u << k;
                if (ts.base) {
                    base[k] = ts.base;
                    goff[k] = uint32_t((row < ts.valid_rows ? row : 0) * ts.row_stride + col);
                }
                f32[k] = ts.to_f32;
                const uint32_t esz = ts.to_f32 ? 4u : uint32_t(sizeof(T));
                dst[k] = ts.lds_off + uint32_t(row * ts.pitch + col) * esz;
            }
        }
    }

    // Issues the loads of a full chunk that starts at t0 (t0 + KT <= L).
    // Every slot loads, from a valid address (unused slots from tile 0), so
    // the loads need no branch.
    __device__ __forceinline__ void fetch_full(int64_t t0) {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            if constexpr (VEC * sizeof(T) == 16) {
                const u32x4 r = ld_global16(base[k] + t0 + goff[k]);
                reg[k][0] = r.x;
                reg[k][1] = r.y;
                reg[k][2] = r.z;
                reg[k][3] = r.w;
            } else {
                const T v = ld_global(base[k] + t0 + goff[k]);
                uint32_t tmp = 0;
                __builtin_memcpy(&tmp, &v, sizeof(T));
                reg[k][0] = tmp;
            }
        }
    }

    // Guarded loads of the ragged chunk that starts at t0 (t0 + KT > L).
    __device__ __forceinline__ void fetch_tail(int64_t t0, int64_t L, int tid) {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const bool on = (live >> k) & 1u;
            const int col = slot_col(tid, k);
            T v[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e++)
                v[e] = (on && t0 + col + e < L) ? ld_global(base[k] + t0 + goff[k] + e) : T(0);
            uint32_t tmp[kWords] = {};
            __builtin_memcpy(tmp, v, sizeof(v));
#pragma unroll
            for (int w = 0; w < kWords; w++) reg[k][w] = tmp[w];
        }
    }

    __device__ __forceinline__ void fetch(int64_t t0, int64_t L, int tid) {
        if (t0 + KT <= L) fetch_full(t0);
        else fetch_tail(t0, L, tid);
    }

    // Writes the prefetched words to LDS.  With zero_dead (uniform) the words
    // of slots that are not live are written as zeros, for tiles whose dead
    // rows are read (the unused state rows of B and C when dstate < 16).
    __device__ __forceinline__ void stash(char *smem, bool zero_dead = false) {
        if (zero_dead) {
#pragma unroll
            for (int k = 0; k < kSlots; k++)
                if (!((live >> k) & 1u))
#pragma unroll
                    for (int w = 0; w < kWords; w++) reg[k][w] = 0u;
        }
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            if (!used[k]) continue;
            T v[VEC];
            __builtin_memcpy(v, reg[k], sizeof(v));
            if (f32[k]) {
                float *d = reinterpret_cast<float *>(smem + dst[k]);
                if constexpr (VEC % 4 == 0) {
#pragma unroll
                    for (int e = 0; e < VEC; e += 4)
                        *reinterpret_cast<float4 *>(d + e) =
                            make_float4(to_f32<T>(v[e]), to_f32<T>(v[e + 1]), to_f32<T>(v[e + 2]),
                                        to_f32<T>(v[e + 3]));
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; e++) d[e] = to_f32<T>(v[e]);
                }
            } else {
                T *d = reinterpret_cast<T *>(smem + dst[k]);
                if constexpr (VEC * sizeof(T) == 16) {
                    Raw16 r;
#pragma unroll
                    for (int w = 0; w < 4; w++) r.w[w] = reg[k][w];
                    *reinterpret_cast<Raw16 *>(d) = r;
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; e++) d[e] = v[e];
                }
            }
        }
    }
};

// Writes a [16 rows][KT] tile of T from LDS to global rows (guarded for the
// ragged tail and for rows past the last channel).
template <typename T, int VEC, int KT, int NTHREADS>
__device__ __forceinline__ void store_tile(T *__restrict__ base, int64_t row_stride,
                                           int valid_rows, int64_t t0, int64_t L,
                                           const T *tile, int tid) {
    constexpr int kVecPerRow = KT / VEC;
    constexpr int kVecs = 16 * kVecPerRow;
#pragma unroll
    for (int k = 0; k < (kVecs + NTHREADS - 1) / NTHREADS; k++) {
        const int slot = tid + k * NTHREADS;
        if (slot < kVecs) {
            const int row = slot / kVecPerRow;
            const int c = (slot % kVecPerRow) * VEC;
            if (row < valid_rows) {
                T *dst = base + row * row_stride + t0 + c;
                const T *s = tile + row * KT + c;
                if (VEC * sizeof(T) == 16 && t0 + c + VEC <= L) {
                    st_global16(dst, *reinterpret_cast<const u32x4 *>(s));
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; e++)
                        if (t0 + c + e < L) dst[e] = s[e];
                }
            }
        }
    }
}

}  // namespace ssk
