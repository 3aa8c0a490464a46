// Device helpers shared by the MonarchAttention kernels (gfx950, wave64).
//
// MFMA operand convention used throughout.  For a 16x16 output tile and a
// 32-wide contraction step, lane l (G = l/16) supplies row (A) or column (B)
// index l%16 and eight contraction "slots" 8G..8G+7, stored as one fragment
// of eight elements.  bf16 fragments feed one v_mfma_f32_16x16x32_bf16; f32
// fragments feed eight v_mfma_f32_16x16x4_f32, call j taking slot j of every
// lane group.  Either way A slot (G,j) meets B slot (G,j), so any fixed map
// from slots to contraction indices works as long as both operands use it.
// The output tile gives lane l the rows 4G+i (i = 0..3) of column l%16.
//
// Slot permutation: when an output tile feeds the next product as an
// operand (the softmax weights), the first product loads its A rows in the
// order perm(ct, m) = 8*(m/4) + 4*ct + m%4 for the two 16-row halves ct of a
// 32-row block.  Lane group G then holds rows 8G..8G+7 of the block, which
// is exactly the slot map "slot j <-> index 8G+j" of the next product, and
// the other operand of that product reads eight consecutive elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 storage

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte access
  using frag = bf16x8;
  __device__ static inline frag zero() { return frag{}; }
  __device__ static inline frag ones() {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(1.0f);
    return r;
  }
  __device__ static inline frag load(const bf16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline bf16_t from_f32(float x) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
  }
  __device__ static inline float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
  }
  // eight floats -> fragment (round to nearest even)
  __device__ static inline frag pack(const float* v) {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(v[j]);
    return r;
  }
  // eight floats (already in output order) -> one 16-byte store
  __device__ static inline void store8(bf16_t* p, const float* v) {
    frag r = pack(v);
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, r);
  }
  __device__ static inline void store4(bf16_t* p, const float* v) {
    uint2 u;
    u.x = static_cast<uint32_t>(from_f32(v[0])) | (static_cast<uint32_t>(from_f32(v[1])) << 16);
    u.y = static_cast<uint32_t>(from_f32(v[2])) | (static_cast<uint32_t>(from_f32(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
  // the value a fragment slot holds, as float (for sums of rounded weights)
  __device__ static inline float slot(const frag& f, int j) { return static_cast<float>(f[j]); }
};

template <> struct Elem<float> {
  static constexpr int kVec = 4;
  struct frag { f32x4 lo, hi; };
  __device__ static inline frag zero() { return frag{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ static inline frag ones() { return frag{f32x4{1, 1, 1, 1}, f32x4{1, 1, 1, 1}}; }
  __device__ static inline frag load(const float* p) {
    frag r;
    r.lo = *reinterpret_cast<const f32x4*>(p);
    r.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return r;
  }
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
    return c;
  }
  __device__ static inline float from_f32(float x) { return x; }
  __device__ static inline float to_f32(float x) { return x; }
  __device__ static inline frag pack(const float* v) {
    frag r;
#pragma unroll
    for (int j = 0; j < 4; ++j) { r.lo[j] = v[j]; r.hi[j] = v[4 + j]; }
    return r;
  }
  __device__ static inline void store8(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  __device__ static inline void store4(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
  __device__ static inline float slot(const frag& f, int j) { return j < 4 ? f.lo[j] : f.hi[j - 4]; }
};


// LDS tiles: rows of DK elements with no padding; the 16-byte chunks of row r
// are stored XOR-permuted by swz(r) = 4*(r%4) + (r/8)%4 (masked to the row's
// chunk count).  Both read patterns below then spread each 16-lane group over
// all banks: row reads (16 rows that differ in bits 0,1,3,4, same chunk) and
// transposing reads (4 consecutive rows x 4 consecutive chunks).
template <typename T, int DK>
struct Tile {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int NCH = DK / V;
  __device__ static inline int swz(int r) { return (4 * (r & 3) + ((r >> 3) & 3)) & (NCH - 1); }
  // element offset of (row r, column col)
  __device__ static inline int off(int r, int col) {
    return r * DK + (((col / V) ^ swz(r)) * V) + (col % V);
  }
  // eight consecutive elements of row r from column col (col % 8 == 0)
  __device__ static inline typename Elem<T>::frag load8(const T* t, int r, int col) {
    if constexpr (V == 8) {
      return Elem<T>::load(t + off(r, col));
    } else {
      typename Elem<T>::frag f;
      f.lo = *reinterpret_cast<const f32x4*>(t + off(r, col));
      f.hi = *reinterpret_cast<const f32x4*>(t + off(r, col + 4));
      return f;
    }
  }
  // Fragment whose contraction index runs down the rows: lane (G, i) gets
  // t[k0 + 8G + j][cbase + cstride*(i/4) + i%4], j = 0..7.
  __device__ static inline typename Elem<T>::frag load_tr(const T* t, int k0, int cbase, int cstride) {
    const int l = threadIdx.x & 63;
    const int i = l & 15, G = l >> 4;
    if constexpr (V == 8) {
      // two ds_read_b64_tr_b16: within each 16-lane block, output lane i,
      // element j is element i%4 of the 8 bytes addressed by lane 4j + i/4
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef short v8i16 __attribute__((ext_vector_type(8)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const int r = k0 + 8 * G + (i >> 2);
      const int col = cbase + cstride * (i & 3);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + off(r, col)));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + off(r + 4, col)));
      const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(typename Elem<T>::frag, v);
    } else {
      const int col = cbase + cstride * (i >> 2) + (i & 3);
      typename Elem<T>::frag f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f.lo[j] = t[off(k0 + 8 * G + j, col)];
        f.hi[j] = t[off(k0 + 8 * G + 4 + j, col)];
      }
      return f;
    }
  }
  // Half of it for a 16-row block (2-byte elements): lane (G, i) gets
  // t[k0 + 4G + j][cbase + cstride*(i/4) + i%4] in slot j = 0..3 and zeros
  // in slots 4..7, so contraction slot 8G + j holds row 4G + j.
  __device__ static inline typename Elem<T>::frag load_tr_half(const T* t, int k0, int cbase, int cstride) {
    static_assert(V == 8, "2-byte elements only");
    const int l = threadIdx.x & 63;
    const int i = l & 15, G = l >> 4;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int r = k0 + 4 * G + (i >> 2);
    const int col = cbase + cstride * (i & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + off(r, col)));
    const v4i16 zero = {0, 0, 0, 0};
    const v8i16 v = __builtin_shufflevector(lo, zero, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Elem<T>::frag, v);
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

// Row of a 32-row block that row slot m of half ct loads (see header).
__device__ inline int perm_row(int ct, int m) { return 8 * (m >> 2) + 4 * ct + (m & 3); }

// Bounds of tile g of the a1 index: floor(g*b1/t).
__device__ inline int tile_lo(int g, int b1, int t) {
  return static_cast<int>((static_cast<long long>(g) * b1) / t);
}

// Spread consecutive logical work items over one XCD: the hardware hands
// workgroup i to XCD i % 8, so items that share inputs through L2 get
// consecutive logical ids on the same XCD.
__device__ inline int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  const int per = nblocks / kXcd, rem = nblocks % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Register-staged copy of a ROWS x DK tile (row stride `rstride` elements in
// global memory) into a swizzled LDS Tile.  load() issues the global reads;
// store() writes them to LDS, so a caller can compute on one LDS buffer while
// the next tile is in flight.  Rows >= nvalid and columns >= D (up to DK) are
// zero.
template <typename T, int D, int DK, int ROWS, int NT>
struct TileLoader {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int VPR = DK / V;
  static constexpr int TOTAL = ROWS * VPR;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint4 buf[PER];
  __device__ inline void load(const T* g, long long rstride, int nvalid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int r = idx / VPR, c = (idx % VPR) * V;
      buf[u] = uint4{0u, 0u, 0u, 0u};
      if ((TOTAL % NT == 0 || idx < TOTAL) && r < nvalid && c < D)
        buf[u] = *reinterpret_cast<const uint4*>(g + r * rstride + c);
    }
  }
  __device__ inline void store(T* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (TOTAL % NT != 0 && idx >= TOTAL) break;
      const int r = idx / VPR, c = (idx % VPR) * V;
      *reinterpret_cast<uint4*>(lds + Tile<T, DK>::off(r, c)) = buf[u];
    }
  }
};


// Global -> LDS DMA of a ROWS x DK tile (row stride `rstride` elements) into a
// swizzled Tile.  One wave instruction writes 1 KiB of consecutive LDS bytes,
// lane l 16 bytes at base + 16*l (measured on gfx950), so each lane fetches
// the global chunk that belongs at its LDS position.  Rows >= nvalid are read
// from row nvalid-1 and columns >= D (only D = 16 with DK = 32) from column
// col - D: finite data that callers give zero weight (rows) or multiply by
// zero contraction slots (columns).  Completion is tracked by vmcnt; callers
// wait (a __syncthreads waits for everything) before reading the tile.
template <typename T, int D, int DK, int ROWS, int NW>
struct TileDma {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int ROWB = DK * static_cast<int>(sizeof(T));
  static constexpr int NINS = ROWS * ROWB / 1024;
  static_assert(NINS * 1024 == ROWS * ROWB, "tile must be a whole number of KiB");
  // The source offset of a lane within the tile fits 32 bits (ROWS rows of
  // at most kMaxB2 * 128 elements), so it is formed in 32-bit arithmetic and
  // added to the wave-uniform base once: the load then takes a scalar base
  // and a 32-bit lane offset, with no 64-bit multiply per lane.
  __device__ static inline void issue(T* tile, const T* g, long long rstride, int nvalid) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const unsigned rs = static_cast<unsigned>(rstride);
    const char* gb = reinterpret_cast<const char*>(g);
#pragma unroll
    for (int i = 0; i < (NINS + NW - 1) / NW; ++i) {
      const int ci = wave + i * NW;
      if (NINS % NW != 0 && ci >= NINS) break;
      const int byte = ci * 1024 + 16 * lane;
      const int r = byte / ROWB;
      const int c = ((byte % ROWB) / 16) ^ Tile<T, DK>::swz(r);  // logical chunk at this position
      int col = c * V;
      if (col >= D) col -= D;
      const unsigned rr = static_cast<unsigned>(r < nvalid ? r : nvalid - 1);
      const unsigned off = (rr * rs + static_cast<unsigned>(col)) * static_cast<unsigned>(sizeof(T));
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(gb + off),
                                       (__attribute__((address_space(3))) void*)(tile + ci * (1024 / static_cast<int>(sizeof(T)))),
                                       16, 0, 0);
    }
  }

  // The lane's byte offsets for a whole tile of row stride `rstride`, formed
  // once per kernel: a streaming loop then issues each whole tile with no
  // per-lane address arithmetic (only the last, partial tile clamps rows).
  static constexpr int PER = (NINS + NW - 1) / NW;
  struct Plan {
    unsigned off[PER];
  };
  __device__ static inline Plan plan(long long rstride) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    Plan pl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ci = wave + i * NW;
      const int byte = ci * 1024 + 16 * lane;
      const int r = byte / ROWB;
      const int c = ((byte % ROWB) / 16) ^ Tile<T, DK>::swz(r);
      int col = c * V;
      if (col >= D) col -= D;
      pl.off[i] = (static_cast<unsigned>(r) * static_cast<unsigned>(rstride) + static_cast<unsigned>(col)) *
                  static_cast<unsigned>(sizeof(T));
    }
    return pl;
  }
  __device__ static inline void issue(T* tile, const T* g, const Plan& pl, long long rstride, int nvalid) {
    if (nvalid < ROWS) {
      issue(tile, g, rstride, nvalid);
      return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const char* gb = reinterpret_cast<const char*>(g);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ci = wave + i * NW;
      if (NINS % NW != 0 && ci >= NINS) break;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(gb + pl.off[i]),
                                       (__attribute__((address_space(3))) void*)(tile + ci * (1024 / static_cast<int>(sizeof(T)))),
                                       16, 0, 0);
    }
  }
};

// Global -> LDS DMA of 64 floats, one per lane of the calling wave:
// dst[l] = src[min(l, nvalid - 1) * stride].
__device__ inline void dma_floats64(float* dst, const float* src, long long stride, int nvalid) {
  const int lane = threadIdx.x & 63;
  const unsigned rr = static_cast<unsigned>(lane < nvalid ? lane : nvalid - 1);
  const unsigned off = rr * static_cast<unsigned>(stride) * 4u;  // < 2^32: 64 rows of a stride <= kMaxB2
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const char*>(src) + off),
                                   (__attribute__((address_space(3))) void*)(dst), 4, 0, 0);
}



}  // namespace monarch
