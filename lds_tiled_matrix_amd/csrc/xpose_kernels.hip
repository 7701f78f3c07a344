// LDS-tiled out-of-place transpose for gfx950 (CDNA4, 64-lane wavefronts).
//
// Method ("Shared memory and the bank conflict", section "Turn the tile
// around on chip"): each workgroup reads one tile of the input with coalesced
// row accesses, stores it into an on-chip tile, waits at one barrier, reads
// the tile back column-wise and writes the columns out as coalesced rows of
// the output.  The barrier is the only synchronisation: the second phase
// reads words other waves wrote in the first (same page, "The barrier").
//
// What is re-derived for gfx950 rather than taken from the pages:
//  * Global side: every lane moves 16 bytes per access (global_load_dwordx4 /
//    global_store_dwordx4), so a run of 8 lanes covers one 128-byte line of a
//    tile row; the pages' kernel moves 4 bytes per lane.
//  * LDS unit: the tile is held as 32-bit words ("units").  1- and 2-byte
//    elements are packed VERTICALLY, K = 4/size input rows of one column per
//    word, by an in-register K x K byte transpose before the LDS write.  The
//    column walk of the second phase then gathers whole words that are
//    already output-ordered, so every element size reduces to the same word
//    tile.  8-byte elements use 64-bit units.
//  * Bank mapping: the column walk is the conflict site ("Shared Memory and
//    Bank Conflicts", "the classic case").  On 64-lane hardware conflicts are
//    resolved per group of lanes whose size must be measured ("the wave size
//    complication"), so the lane maps below never let one 32-lane half-wave
//    span more than eight 16-byte chunks of a tile row; with a one-word pad
//    or a 16-byte XOR swizzle the column read is then conflict-free whether
//    the hardware resolves 32 lanes over 32 banks or 64 lanes over 64 banks.
//  * Edges: tiles that cross the matrix edge (or matrices whose rows are not
//    4-byte aligned) take an element-wise path through the same LDS tile;
//    nothing outside the logical output is written.
//  * Variants, each measured against the default: persistent double-buffered
//    workgroups, direct global->LDS loads, 1- and 2-byte tiles read back
//    with the LDS transpose reads, line-aligned output tiles for output rows
//    off the 128-byte line, and two naive kernels without LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "xpose_kernels.h"
#include "xpose_lanes.h"

namespace xpose {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global access at any byte address.  Under the ROCm runtime the
// gfx9 family runs in unaligned-access mode and global_load/store_dwordx4
// take any address (the memory pipeline splits an access that straddles
// cache lines), so rows whose pitch is an odd number of 1-, 2- or 4-byte
// elements still take one 16-byte access per lane.  (Direct global->LDS
// loads are the exception: their rows must be 4-byte aligned.)
typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(1)));

template <int CP>
__device__ __forceinline__ u32x4 load16(const char *p) {
  const u32x4u *q = reinterpret_cast<const u32x4u *>(p);
  if constexpr (CP == kNtLoadStore) return __builtin_nontemporal_load(q);
  else return *q;
}

template <int CP>
__device__ __forceinline__ void store16(char *p, u32x4 x) {
  u32x4u *q = reinterpret_cast<u32x4u *>(p);
  if constexpr (CP != kCacheDefault) __builtin_nontemporal_store((u32x4u)x, q);
  else *q = x;
}


// K input-row vectors (16 bytes each, same columns) -> V column units.
// Unit e holds column e of the K rows, first row in the lowest bytes.
template <int S>
__device__ __forceinline__ void pack_units(const u32x4 *rows,
                                           typename Elem<S>::U *u) {
  if constexpr (S == 4) {
    u[0] = rows[0].x; u[1] = rows[0].y; u[2] = rows[0].z; u[3] = rows[0].w;
  } else if constexpr (S == 8) {
    u[0] = (uint64_t)rows[0].x | ((uint64_t)rows[0].y << 32);
    u[1] = (uint64_t)rows[0].z | ((uint64_t)rows[0].w << 32);
  } else if constexpr (S == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = rows[0][j], b = rows[1][j];
      u[2 * j] = (a & 0xFFFFu) | (b << 16);
      u[2 * j + 1] = (a >> 16) | (b & 0xFFFF0000u);
    }
  } else {  // S == 1: 4 x 4 byte transpose per word column
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int sh = 8 * b;
        u[4 * j + b] = ((rows[0][j] >> sh) & 0xFFu) |
                       (((rows[1][j] >> sh) & 0xFFu) << 8) |
                       (((rows[2][j] >> sh) & 0xFFu) << 16) |
                       (((rows[3][j] >> sh) & 0xFFu) << 24);
      }
    }
  }
}

// UPV units gathered down one LDS column -> one 16-byte output vector.
template <int S>
__device__ __forceinline__ u32x4 units_to_vec(const typename Elem<S>::U *u) {
  if constexpr (S == 8) {
    return u32x4{(uint32_t)u[0], (uint32_t)(u[0] >> 32), (uint32_t)u[1],
                 (uint32_t)(u[1] >> 32)};
  } else {
    return u32x4{u[0], u[1], u[2], u[3]};
  }
}

// Store the V units one load task produced: row p, columns c .. c+V-1.
template <class T>
__device__ __forceinline__ void write_units(typename T::U *lds, int p, int c,
                                            const typename T::U *u) {
  if constexpr (T::WIDE_WRITE) {
#pragma unroll
    for (int g = 0; g < T::V / T::UPV; ++g) {
      const int idx = T::lds_index(p, c + g * T::UPV);
      if constexpr (T::UB == 4) {
        *reinterpret_cast<u32x4 *>(lds + idx) =
            u32x4{u[4 * g], u[4 * g + 1], u[4 * g + 2], u[4 * g + 3]};
      } else {
        *reinterpret_cast<u32x4 *>(lds + idx) =
            u32x4{(uint32_t)u[2 * g], (uint32_t)(u[2 * g] >> 32),
                  (uint32_t)u[2 * g + 1], (uint32_t)(u[2 * g + 1] >> 32)};
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < T::V; ++e) lds[T::lds_index(p, c + e)] = u[e];
  }
}

// Gather one output vector: units (q*UPV + k, c) for k < UPV.
template <class T>
__device__ __forceinline__ u32x4 read_column(const typename T::U *lds, int c,
                                             int q) {
  typename T::U u[T::UPV];
#pragma unroll
  for (int k = 0; k < T::UPV; ++k) u[k] = lds[T::lds_index(q * T::UPV + k, c)];
  return units_to_vec<sizeof(typename T::E)>(u);
}

// Interior tile, rows 4-byte aligned: 128-bit global accesses throughout.
// Split in three so the persistent kernel can keep the next tile's loads in
// flight while it drains the current one.
template <class T>
struct TileRegs {
  u32x4 v[T::LIT][T::K];
};

// Phase 1a: 16-byte row loads of one tile into registers.
template <class T>
__device__ __forceinline__ void vector_load(const char *src, int64_t ld_in,
                                            int wave, int lane,
                                            TileRegs<T> &r) {
  constexpr int S = (int)sizeof(typename T::E);
  constexpr bool LSPLIT = !T::WIDE_WRITE;
#pragma unroll
  for (int it = 0; it < T::LIT; ++it) {
    int p, ch;
    lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
#pragma unroll
    for (int k = 0; k < T::K; ++k)
      r.v[it][k] = load16<T::CACHE>(
          src + ((int64_t)(p * T::K + k) * ld_in + ch * T::V) * S);
  }
}

// Phase 1b: registers -> LDS tile (after the K x K packing).
template <class T>
__device__ __forceinline__ void vector_to_lds(typename T::U *lds,
                                              const TileRegs<T> &r, int wave,
                                              int lane) {
  constexpr int S = (int)sizeof(typename T::E);
  constexpr bool LSPLIT = !T::WIDE_WRITE;
#pragma unroll
  for (int it = 0; it < T::LIT; ++it) {
    int p, ch;
    lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
    typename T::U u[T::V];
    pack_units<S>(r.v[it], u);
    write_units<T>(lds, p, ch * T::V, u);
  }
}

// Phase 2: column gathers from LDS -> 16-byte row stores.
template <class T>
__device__ __forceinline__ void lds_to_global(const typename T::U *lds,
                                              char *dst, int64_t ld_out,
                                              int wave, int lane) {
  constexpr int S = (int)sizeof(typename T::E);
#pragma unroll
  for (int it = 0; it < T::SIT; ++it) {
    int c, q;
    lane_map<T::NCO, true>(it * T::NW + wave, lane, c, q);
    const u32x4 o = read_column<T>(lds, c, q);
    store16<T::CACHE>(dst + ((int64_t)c * ld_out + q * T::V) * S, o);
  }
}

// Phase 1, direct variant (4- and 8-byte elements, rows contiguous in LDS):
// one global_load_lds_dwordx4 per wave task puts the 64 lanes' 16 bytes at
// 64 consecutive 16-byte slots of LDS, slot l for lane l.  Lane l therefore
// fetches the logical chunk that belongs in physical slot l: the swizzle is
// applied to the global address instead of the LDS address (XOR is its own
// inverse).  The permutation stays inside one tile row, so each row's loads
// remain one contiguous, coalesced range.
template <class T>
__device__ __forceinline__ void direct_load_to_lds(typename T::U *lds,
                                                   const char *src,
                                                   int64_t ld_in, int wave,
                                                   int lane) {
  constexpr int S = (int)sizeof(typename T::E);
  constexpr int RPW = 64 / T::NCI;  // tile rows per wave task
#pragma unroll
  for (int it = 0; it < T::LIT; ++it) {
    const int wt = it * T::NW + wave;
    const int p = wt * RPW + lane / T::NCI;
    const int slot = lane % T::NCI;
    int chunk = slot;
    if constexpr (T::LAYOUT == kSwizzle) chunk = slot ^ T::chunk_xor(p, 0);
    const char *g = src + ((int64_t)p * ld_in + chunk * T::V) * S;
    __builtin_amdgcn_global_load_lds(
        g, (__attribute__((address_space(3))) void *)(lds + wt * RPW * T::TCOLS),
        16, 0, 0);
  }
  // The data reaches LDS through the vector-memory path: wait for it before
  // the barrier publishes the tile.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class T>
__device__ __forceinline__ void tile_vector(typename T::U *lds, const char *src,
                                            char *dst, int64_t ld_in,
                                            int64_t ld_out, int wave,
                                            int lane) {
  if constexpr (T::DIRECT_LDS) {
    direct_load_to_lds<T>(lds, src, ld_in, wave, lane);
  } else {
    TileRegs<T> r;
    vector_load<T>(src, ld_in, wave, lane, r);
    vector_to_lds<T>(lds, r, wave, lane);
  }
  __syncthreads();
  lds_to_global<T>(lds, dst, ld_out, wave, lane);
}

// Edge tile: the same LDS tile and lane maps, with every global access
// bounds-checked against the rows and columns left in the matrix.  With VEC
// (the call may use 16-byte accesses) each whole 16-byte chunk or vector
// inside the matrix still moves as one access and only the pieces that cross
// the edge go element by element; without it (the element-wise path asked
// for explicitly, or rows a direct-load kernel cannot take) every access is
// one element.
// Phase 1 of an edge tile on the 16-byte path, every load issued before the
// first wait: each chunk is one unconditional 16-byte load from an address
// chosen without a branch (a branch around each load makes the compiler
// wait for every load before it issues the next).  edge_chunk_src and
// edge_chunk_fix in xpose_lanes.h state the same address choice and fix-up
// as host functions, which a host test checks against a guard page.
//  * whole chunk inside the matrix: the chunk itself;
//  * chunk across the row's end (partial): the 16 bytes that END at the
//    row's last element, then shifted down so the chunk's elements come
//    first and the bytes past the row's end are zero.  Those 16 bytes lie in
//    the row because the tile holds at least V columns (cols_left >= V);
//  * chunk past the row's end, or row past the matrix: the tile's first
//    chunk (whole, by the same condition), then zeroed.
template <class T>
__device__ __forceinline__ void edge_load_batched(typename T::U *lds,
                                                  const char *src,
                                                  int64_t ld_in,
                                                  int64_t rows_left,
                                                  int64_t cols_left, int wave,
                                                  int lane) {
  constexpr int S = (int)sizeof(typename T::E);
  constexpr bool LSPLIT = !T::WIDE_WRITE;
  u32x4 v[T::LIT][T::K];
#pragma unroll
  for (int it = 0; it < T::LIT; ++it) {
    int p, ch;
    lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
    const int64_t have = cols_left - (int64_t)ch * T::V;  // elements left
#pragma unroll
    for (int k = 0; k < T::K; ++k) {
      const int row = p * T::K + k;
      const char *rs = src + ((int64_t)row * ld_in + ch * T::V) * S;
      const char *at = src;
      if (row < rows_left && have > 0)
        at = have >= T::V ? rs : rs + have * S - 16;
      v[it][k] = load16<T::CACHE>(at);
    }
  }
#pragma unroll
  for (int it = 0; it < T::LIT; ++it) {
    int p, ch;
    lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
    const int64_t have = cols_left - (int64_t)ch * T::V;
#pragma unroll
    for (int k = 0; k < T::K; ++k) {
      const int row = p * T::K + k;
      if (row >= rows_left || have <= 0) {
        v[it][k] = u32x4{0, 0, 0, 0};
      } else if (have < T::V) {
        // bytes [16 - have * S, 16) of the load are the chunk's first
        // have * S bytes: shift the 128-bit value down by that offset.
        const int sh = (int)(16 - have * S) * 8;  // 8 .. 120 bits
        uint64_t lo = (uint64_t)v[it][k].x | ((uint64_t)v[it][k].y << 32);
        uint64_t hi = (uint64_t)v[it][k].z | ((uint64_t)v[it][k].w << 32);
        if (sh >= 64) {
          lo = hi >> (sh - 64);
          hi = 0;
        } else {
          lo = (lo >> sh) | (hi << (64 - sh));
          hi >>= sh;
        }
        v[it][k] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                         (uint32_t)(hi >> 32)};
      }
    }
    typename T::U u[T::V];
    pack_units<S>(v[it], u);
    write_units<T>(lds, p, ch * T::V, u);
  }
}

template <class T, bool VEC>
__device__ __forceinline__ void tile_elementwise(typename T::U *lds,
                                                 const char *src, char *dst,
                                                 int64_t ld_in, int64_t ld_out,
                                                 int64_t rows_left,
                                                 int64_t cols_left, int wave,
                                                 int lane) {
  using E = typename T::E;
  constexpr int S = (int)sizeof(E);
  constexpr bool LSPLIT = !T::WIDE_WRITE;
  if (VEC && cols_left >= T::V) {  // uniform per workgroup
    edge_load_batched<T>(lds, src, ld_in, rows_left, cols_left, wave, lane);
  } else {
#pragma unroll
    for (int it = 0; it < T::LIT; ++it) {
      int p, ch;
      lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
      u32x4 v[T::K];
#pragma unroll
      for (int k = 0; k < T::K; ++k) {
        const int row = p * T::K + k;
        const char *rs = src + ((int64_t)row * ld_in + ch * T::V) * S;
        if (VEC && row < rows_left && (ch + 1) * T::V <= cols_left) {
          v[k] = load16<T::CACHE>(rs);
        } else if (VEC && S <= 2) {
          // 1- and 2-byte elements: the chunk's elements inside the matrix
          // in at most four pieces instead of up to 16 element loads.
          const int64_t have = row < rows_left ? cols_left - ch * T::V : 0;
          uint64_t lo, hi;
          load_head(rs, have > 0 ? (int)(have * S) : 0, lo, hi);
          v[k] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                       (uint32_t)(hi >> 32)};
        } else {
          E e[T::V];
#pragma unroll
          for (int x = 0; x < T::V; ++x)
            e[x] = (row < rows_left && ch * T::V + x < cols_left)
                       ? reinterpret_cast<const E *>(rs)[x]
                       : E(0);
          __builtin_memcpy(&v[k], e, 16);
        }
      }
      typename T::U u[T::V];
      pack_units<S>(v, u);
      write_units<T>(lds, p, ch * T::V, u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < T::SIT; ++it) {
    int c, q;
    lane_map<T::NCO, true>(it * T::NW + wave, lane, c, q);
    const u32x4 o = read_column<T>(lds, c, q);
    if (c < cols_left) {
      char *d = dst + ((int64_t)c * ld_out + q * T::V) * S;
      if (VEC && (q + 1) * T::V <= rows_left) {
        store16<T::CACHE>(d, o);
      } else if (VEC && S <= 2) {
        const int64_t have = rows_left - q * T::V;
        store_head(d, have > 0 ? (int)(have * S) : 0,
                   (uint64_t)o.x | ((uint64_t)o.y << 32),
                   (uint64_t)o.z | ((uint64_t)o.w << 32));
      } else {
        E e[T::V];
        __builtin_memcpy(e, &o, 16);
#pragma unroll
        for (int x = 0; x < T::V; ++x)
          if (q * T::V + x < rows_left) reinterpret_cast<E *>(d)[x] = e[x];
      }
    }
  }
}

template <class T>
__device__ __forceinline__ void tile_edge(bool vec_ok, typename T::U *lds,
                                          const char *src, char *dst,
                                          int64_t ld_in, int64_t ld_out,
                                          int64_t rows_left, int64_t cols_left,
                                          int wave, int lane) {
  // vec_ok is uniform over the launch, so every wave takes the same branch
  // and reaches the barrier inside.
  if (vec_ok)
    tile_elementwise<T, true>(lds, src, dst, ld_in, ld_out, rows_left,
                              cols_left, wave, lane);
  else
    tile_elementwise<T, false>(lds, src, dst, ld_in, ld_out, rows_left,
                               cols_left, wave, lane);
}

// Where one tile lives.
struct TileSpot {
  const char *src;
  char *dst;
  int64_t rows_left, cols_left;
  bool vec;  // interior tile on the 128-bit path
};

template <int S, int TR, int TC>
__device__ __forceinline__ TileSpot tile_spot(const TileArgs &a, uint32_t t,
                                              uint32_t ntiles) {
  uint32_t tr, tc;
  int64_t b;
  tile_coords(a, t, ntiles, tr, tc, b);
  const int64_t r0 = (int64_t)tr * TR, c0 = (int64_t)tc * TC;
  TileSpot p;
  p.src = static_cast<const char *>(a.in) +
          (b * a.stride_in + r0 * a.ld_in + c0) * S;
  p.dst = static_cast<char *>(a.out) +
          (b * a.stride_out + c0 * a.ld_out + r0) * S;
  p.rows_left = a.rows - r0;
  p.cols_left = a.cols - c0;
  p.vec = a.vec_ok && p.rows_left >= TR && p.cols_left >= TC;
  return p;
}

// One tile per workgroup.
template <int S, int TR, int TC, int NT, int L, int CP, bool DIRECT = false>
__global__ __launch_bounds__(NT) void xpose_tile_kernel(TileArgs a) {
  using T = Tile<S, TR, TC, NT, L, CP, DIRECT>;
  __shared__ __attribute__((aligned(16))) typename T::U lds[T::LDS_UNITS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const TileSpot p = tile_spot<S, TR, TC>(a, blockIdx.x, gridDim.x);
  // Uniform per workgroup, so the barrier inside either path is reached by
  // every wave of the block.
  if (p.vec)
    tile_vector<T>(lds, p.src, p.dst, a.ld_in, a.ld_out, wave, lane);
  else
    tile_edge<T>(a.vec_ok, lds, p.src, p.dst, a.ld_in, a.ld_out, p.rows_left,
                 p.cols_left, wave, lane);
}

// Persistent workgroups: workgroup w handles tiles w, w + G, w + 2G, ... of
// `ntiles` (G = gridDim.x, a multiple of 8 so every tile stays on the XCD the
// per-XCD remap assigns it to).  Two LDS buffers alternate between
// consecutive tiles, and the next tile's loads are issued right after the
// current tile's barrier, so they are in flight while the current tile is
// gathered and stored.  One barrier per tile is enough: buffer b is written
// again two tiles later, after the intervening tile's barrier, which every
// wave reaches only once it has finished reading b (the overwrite-before-
// last-read hazard of "Shared-memory tiling and bank conflicts", section
// "Protect tile phases and account for capacity").
template <int S, int TR, int TC, int NT, int L, int CP>
__global__ __launch_bounds__(NT) void xpose_tile_persistent_kernel(
    TileArgs a, uint32_t ntiles) {
  using T = Tile<S, TR, TC, NT, L, CP>;
  __shared__ __attribute__((aligned(16))) typename T::U lds[2][T::LDS_UNITS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t t = blockIdx.x;
  if (t >= ntiles) return;  // uniform per workgroup
  TileSpot cur = tile_spot<S, TR, TC>(a, t, ntiles);
  TileRegs<T> r;
  if (cur.vec) vector_load<T>(cur.src, a.ld_in, wave, lane, r);
  int buf = 0;
  for (;;) {
    const uint32_t tn = t + gridDim.x;
    const bool more = tn < ntiles;
    TileSpot next;
    if (more) next = tile_spot<S, TR, TC>(a, tn, ntiles);
    if (cur.vec) {
      vector_to_lds<T>(lds[buf], r, wave, lane);
      __syncthreads();
      if (more && next.vec) vector_load<T>(next.src, a.ld_in, wave, lane, r);
      lds_to_global<T>(lds[buf], cur.dst, a.ld_out, wave, lane);
    } else {
      tile_edge<T>(a.vec_ok, lds[buf], cur.src, cur.dst, a.ld_in, a.ld_out,
                   cur.rows_left, cur.cols_left, wave, lane);
      if (more && next.vec) vector_load<T>(next.src, a.ld_in, wave, lane, r);
    }
    if (!more) break;
    cur = next;
    t = tn;
    buf ^= 1;
  }
}

// lds_extra: bytes of dynamic LDS reserved per workgroup and never touched.
// It only raises the workgroup's LDS footprint, which caps how many
// workgroups of the launch share one compute unit.
template <int S, int TR, int TC, int NT, int L, int CP, bool DIRECT = false>
hipError_t launch_tile(const TileArgs &a, uint32_t grid, uint32_t lds_extra,
                       hipStream_t stream) {
  TileArgs copy = a;
  void *args[] = {&copy};
  // hipLaunchKernel reports this launch's own status; the sticky
  // hipGetLastError can hold an unrelated earlier error of the process.
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          &xpose_tile_kernel<S, TR, TC, NT, L, CP, DIRECT>),
      dim3(grid), dim3(NT), args, lds_extra, stream);
}

template <int S, int TR, int TC, int NT, int L, int CP>
hipError_t launch_tile_persistent(const TileArgs &a, uint32_t ntiles,
                                  uint32_t grid, hipStream_t stream) {
  TileArgs copy = a;
  uint32_t n = ntiles;
  void *args[] = {&copy, &n};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          &xpose_tile_persistent_kernel<S, TR, TC, NT, L, CP>),
      dim3(grid), dim3(NT), args, 0, stream);
}

// ---------------------------------------------------------------------------
// Line-aligned output tiles (2-, 4- and 8-byte elements).  When output rows
// do not start on a 128-byte line, a tile's output segments [r0, r0 + TR)
// straddle lines at both ends; non-temporal writes of such partial lines go
// to memory as partial lines.  Here each tile shifts its segment in output
// row j back by
//   d_j = (byte address of output row j mod 128) / S   (elements, < 128 / S),
// so the segment [r0 - d_j, r0 - d_j + TR) starts on a line and is whole
// lines.  Over tile rows tr = 0 .. tiles_r - 1, with tiles_r = ceil((rows +
// 128 / S - 1) / TR), the shifted segments of each output row partition
// [0, rows).  The LDS tile therefore holds TR + 128 / S input rows, [r0 -
// 128 / S, r0 + TR): a halo of one line above the tile, which the previous
// tile row has just read (the super-tile order walks tile rows fastest).
// For 2-byte elements, packed two rows per 32-bit unit, a segment starting
// at an odd row takes each output word from two units (shift_gather).
// ---------------------------------------------------------------------------

template <class T>
__device__ __forceinline__ u32x4 shift_gather(const typename T::U *lds,
                                              int rel, int c) {
  int ur, shift;
  T::gather_rows(rel, ur, shift);
  typename T::U w[T::GATHER_UNITS];
#pragma unroll
  for (int k = 0; k < T::GATHER_UNITS; ++k)
    w[k] = lds[T::unit_index(ur + k, c)];
  if constexpr (T::K == 1) {
    return units_to_vec<sizeof(typename T::Base::E)>(w);
  } else {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], shift);
    return o;
  }
}

// Phase 1 of a line-aligned tile: input rows [top, top + PR) x columns
// [c0, c0 + TC) into the swizzled LDS tile, rows outside the matrix and
// columns past its edge as zero (never stored).  Three load paths, chosen
// per workgroup:
//  * kShiftInner (every row and chunk inside the matrix): no checks, so
//    each lane issues all its loads before it waits for the first;
//  * kShiftEdge (some row or chunk outside, but the tile holds at least V
//    columns): as the edge tiles' edge_load_batched, every chunk is one
//    unconditional 16-byte load from an address picked without a branch --
//    the chunk; the 16 bytes ending at the row's last element, shifted
//    down; or the tile's first chunk of its first row inside the matrix
//    (row max(top, 0), which the halo keeps below `rows`), zeroed;
//  * kShiftChecked (fewer than V columns): element by element.  There each
//    load sits in its own branch, and the compiler waits for it before the
//    next one is issued.
enum ShiftLoad : int { kShiftInner = 0, kShiftEdge = 1, kShiftChecked = 2 };
template <class T, int MODE>
__device__ __forceinline__ void shift_load(typename T::Base::U *lds,
                                           const char *in, int64_t top,
                                           int64_t rows, int64_t ld_in,
                                           int64_t c0, int64_t cols_left,
                                           int wave, int lane) {
  using B = typename T::Base;
  using E = typename B::E;
  constexpr int S = (int)sizeof(E);
  constexpr int LCP = B::CACHE == kNtLoadStore ? kNtLoadStore : kCacheDefault;
  const char *first = in + ((top > 0 ? top : 0) * ld_in + c0) * S;
  u32x4 v[B::LIT][T::K];
#pragma unroll
  for (int it = 0; it < B::LIT; ++it) {
    int p, ch;
    lane_map<B::NCI, false>(it * B::NW + wave, lane, p, ch);
    const int64_t have = cols_left - (int64_t)ch * T::V;  // elements left
#pragma unroll
    for (int k = 0; k < T::K; ++k) {
      const int64_t row = top + p * T::K + k;
      const char *src = in + (row * ld_in + c0 + ch * T::V) * S;
      if (MODE == kShiftInner) {
        v[it][k] = load16<LCP>(src);
      } else if (MODE == kShiftEdge) {
        const char *at = first;
        if (row >= 0 && row < rows && have > 0)
          at = have >= T::V ? src : src + have * S - 16;
        v[it][k] = load16<LCP>(at);
      } else if (row < 0 || row >= rows) {
        v[it][k] = u32x4{0, 0, 0, 0};
      } else if ((ch + 1) * T::V <= cols_left) {
        v[it][k] = load16<LCP>(src);
      } else {
        E e[T::V];
#pragma unroll
        for (int x = 0; x < T::V; ++x)
          e[x] = ch * T::V + x < cols_left ? reinterpret_cast<const E *>(src)[x]
                                           : E(0);
        __builtin_memcpy(&v[it][k], e, 16);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < B::LIT; ++it) {
    int p, ch;
    lane_map<B::NCI, false>(it * B::NW + wave, lane, p, ch);
    if (MODE == kShiftEdge) {
      const int64_t have = cols_left - (int64_t)ch * T::V;
#pragma unroll
      for (int k = 0; k < T::K; ++k) {
        const int64_t row = top + p * T::K + k;
        if (row < 0 || row >= rows || have <= 0) {
          v[it][k] = u32x4{0, 0, 0, 0};
        } else if (have < T::V) {
          // bytes [16 - have * S, 16) of the load are the chunk's first
          // have * S bytes: shift the 128-bit value down by that offset.
          const int sh = (int)(16 - have * S) * 8;  // 8 .. 120 bits
          uint64_t lo = (uint64_t)v[it][k].x | ((uint64_t)v[it][k].y << 32);
          uint64_t hi = (uint64_t)v[it][k].z | ((uint64_t)v[it][k].w << 32);
          if (sh >= 64) {
            lo = hi >> (sh - 64);
            hi = 0;
          } else {
            lo = (lo >> sh) | (hi << (64 - sh));
            hi >>= sh;
          }
          v[it][k] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                           (uint32_t)(hi >> 32)};
        }
      }
    }
    typename B::U u[T::V];
    pack_units<S>(v[it], u);
    write_units<B>(lds, p, ch * T::V, u);
  }
}

// Phase 2: output row j = c0 + c, line-aligned segment starting at input
// row r0 - d_j; chunk q holds input rows r0 - d_j + V q .. + V - 1, LDS
// input rows HALO - d_j + V q .. (always inside [1, PR)).  INNER: the whole
// segment lies inside the matrix (r0 >= HALO and r0 + TR <= rows) and every
// tile column is a matrix column, so every store is one 16-byte store.
template <class T, int CP, bool INNER>
__device__ __forceinline__ void shift_store(const typename T::Base::U *lds,
                                            char *out, int64_t r0,
                                            int64_t rows, int64_t ld_out,
                                            int64_t c0, int64_t cols_left,
                                            int wave, int lane) {
  using E = typename T::Base::E;
  constexpr int S = (int)sizeof(E);
#pragma unroll
  for (int it = 0; it < T::SIT; ++it) {
    int c, q;
    lane_map<T::NCO, true>(it * T::NW + wave, lane, c, q);
    if (INNER || c < cols_left) {
      char *row_out = out + (c0 + c) * ld_out * S;
      const int d = (int)(((uintptr_t)row_out & 127) / S);
      const int64_t first = r0 - d + T::V * q;  // input row of element 0
      const u32x4 o = shift_gather<T>(lds, T::HALO - d + T::V * q, c);
      if (INNER || (first >= 0 && first + T::V - 1 < rows)) {
        store16<CP>(row_out + first * S, o);
      } else {
        E e[T::V];
        __builtin_memcpy(e, &o, 16);
#pragma unroll
        for (int x = 0; x < T::V; ++x)
          if (first + x >= 0 && first + x < rows)
            reinterpret_cast<E *>(row_out)[first + x] = e[x];
      }
    }
  }
}

template <int S, int TR, int TC, int NT, int CP>
__global__ __launch_bounds__(NT) void xpose_shift_kernel(TileArgs a) {
  using T = ShiftTile<S, TR, TC, NT, CP>;
  using B = typename T::Base;
  __shared__ __attribute__((aligned(16))) typename B::U lds[T::LDS_UNITS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t tr, tc;
  int64_t b;
  tile_coords(a, blockIdx.x, gridDim.x, tr, tc, b);
  const int64_t r0 = (int64_t)tr * TR, c0 = (int64_t)tc * TC;
  const int64_t top = r0 - T::HALO;  // input row of LDS row 0
  const char *in = static_cast<const char *>(a.in) + b * a.stride_in * S;
  char *out = static_cast<char *>(a.out) + b * a.stride_out * S;
  const int64_t cols_left = a.cols - c0;
  // Uniform per workgroup, so every wave takes the same branch and reaches
  // the barrier inside it.
  if (top >= 0 && r0 + TR <= a.rows && cols_left >= TC) {
    shift_load<T, kShiftInner>(lds, in, top, a.rows, a.ld_in, c0, cols_left,
                               wave, lane);
    __syncthreads();
    shift_store<T, CP, true>(lds, out, r0, a.rows, a.ld_out, c0, cols_left,
                             wave, lane);
  } else {
    if (cols_left >= T::V)
      shift_load<T, kShiftEdge>(lds, in, top, a.rows, a.ld_in, c0, cols_left,
                                wave, lane);
    else
      shift_load<T, kShiftChecked>(lds, in, top, a.rows, a.ld_in, c0,
                                   cols_left, wave, lane);
    __syncthreads();
    shift_store<T, CP, false>(lds, out, r0, a.rows, a.ld_out, c0, cols_left,
                              wave, lane);
  }
}

template <int S, int TR, int TC, int NT, int CP>
hipError_t launch_shift(const TileArgs &a, uint32_t grid, uint32_t lds_extra,
                        hipStream_t stream) {
  TileArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(&xpose_shift_kernel<S, TR, TC, NT, CP>),
      dim3(grid), dim3(NT), args, lds_extra, stream);
}

// ---------------------------------------------------------------------------
// Column strips of line-aligned output tiles (4- and 8-byte elements).  The
// one-shot line-aligned tile reads its HALO rows again although the tile
// above it has just read them.  Here workgroup (segment s, tile column tc)
// walks tile rows [s seg, min((s + 1) seg, tiles_r)) of tile column tc top
// to bottom and keeps the input rows in a ring of Q = 2 TR rows of LDS
// (input row r in ring row (r + HALO) mod Q): after the segment's first
// tile, each tile loads only its own TR rows and finds its halo in the
// ring.  The next tile's rows are loaded into registers before the current
// tile is gathered and stored, so those loads are in flight during the
// stores.  Two barriers per tile: every gather of tile t must be done before
// tile t + 1's rows overwrite tile t's halo rows in the ring, and those rows
// must be in the ring before tile t + 1's gathers.  Q is a multiple of the
// swizzle's period, so each ring row keeps the bank pattern of the same row
// of the one-shot tile.
// ---------------------------------------------------------------------------
template <int S, int TR, int TC, int NT, int CP>
struct StripTile {
  using Shift = ShiftTile<S, TR, TC, NT, CP>;
  static constexpr int HALO = Shift::HALO, Q = 2 * TR;
  using Ring = Tile<S, Q, TC, NT, kSwizzle, CP>;
  using U = typename Ring::U;
  static constexpr int V = Ring::V, NCI = Ring::NCI, NW = NT / 64;
  static constexpr int LIT_NEW = TR * NCI / NT;     // load tasks, TR rows
  static constexpr int LIT_HALO = HALO * NCI / NT;  // load tasks, HALO rows
  static constexpr int PERIOD = Ring::UPV * Ring::NCL / Ring::QSTEP;
  static constexpr int LDS_BYTES = Ring::LDS_BYTES;
  static_assert(Ring::K == 1, "one input row per LDS unit (4, 8 bytes)");
  static_assert(HALO <= TR && Q % PERIOD == 0, "ring keeps the swizzle");
  static_assert(LIT_NEW >= 1 && LIT_HALO >= 1 && TR * NCI % NT == 0 &&
                    HALO * NCI % NT == 0,
                "even load split");
  XPOSE_HD static inline int ring_row(int64_t r) {
    return (int)((r + HALO) & (Q - 1));
  }
};

// Input rows [first, first + LIT * NT / NCI) of the strip's columns
// [c0, c0 + TC) into registers; rows outside the matrix and columns past
// its edge read as zero (never stored).  INNER (all of those rows and
// columns inside the matrix): no checks, so the loads go out back to back
// (as in shift_load).
template <class ST, int LIT, bool INNER>
__device__ __forceinline__ void strip_load(u32x4 (&v)[LIT], const char *in,
                                           int64_t first, int64_t rows,
                                           int64_t ld_in, int64_t c0,
                                           int64_t cols_left, int wave,
                                           int lane) {
  constexpr int S = (int)sizeof(typename ST::Ring::E);
  using E = typename Elem<S>::E;
  constexpr int LCP =
      ST::Ring::CACHE == kNtLoadStore ? kNtLoadStore : kCacheDefault;
#pragma unroll
  for (int it = 0; it < LIT; ++it) {
    int p, ch;
    lane_map<ST::NCI, false>(it * ST::NW + wave, lane, p, ch);
    const int64_t row = first + p;
    const char *src = in + (row * ld_in + c0 + ch * ST::V) * S;
    if (INNER) {
      v[it] = load16<LCP>(src);
    } else if (row < 0 || row >= rows) {
      v[it] = u32x4{0, 0, 0, 0};
    } else if ((ch + 1) * ST::V <= cols_left) {
      v[it] = load16<LCP>(src);
    } else {
      E e[ST::V];
#pragma unroll
      for (int x = 0; x < ST::V; ++x)
        e[x] = ch * ST::V + x < cols_left ? reinterpret_cast<const E *>(src)[x]
                                          : E(0);
      __builtin_memcpy(&v[it], e, 16);
    }
  }
}

// strip_load with the checks only where the rows or columns reach past the
// matrix (uniform per workgroup).
template <class ST, int LIT>
__device__ __forceinline__ void strip_load_any(u32x4 (&v)[LIT],
                                               const char *in, int64_t first,
                                               int64_t rows, int64_t ld_in,
                                               int64_t c0, int64_t cols_left,
                                               int wave, int lane) {
  constexpr int64_t N = (int64_t)LIT * ST::Ring::NW * 64 / ST::NCI;
  if (first >= 0 && first + N <= rows && cols_left >= ST::Ring::TCOLS)
    strip_load<ST, LIT, true>(v, in, first, rows, ld_in, c0, cols_left, wave,
                              lane);
  else
    strip_load<ST, LIT, false>(v, in, first, rows, ld_in, c0, cols_left, wave,
                               lane);
}

template <class ST, int LIT>
__device__ __forceinline__ void strip_to_ring(typename ST::U *lds,
                                              const u32x4 (&v)[LIT],
                                              int64_t first, int wave,
                                              int lane) {
  constexpr int S = (int)sizeof(typename ST::Ring::E);
#pragma unroll
  for (int it = 0; it < LIT; ++it) {
    int p, ch;
    lane_map<ST::NCI, false>(it * ST::NW + wave, lane, p, ch);
    typename ST::U u[ST::V];
    pack_units<S>(&v[it], u);
    write_units<typename ST::Ring>(lds, ST::ring_row(first + p), ch * ST::V,
                                   u);
  }
}

// One tile of a strip, gathered from the ring and stored: as shift_store,
// with the unit rows read through the ring.
template <class ST, int CP, bool INNER>
__device__ __forceinline__ void strip_store(const typename ST::U *lds,
                                            char *out, int64_t r0,
                                            int64_t rows, int64_t ld_out,
                                            int64_t c0, int64_t cols_left,
                                            int wave, int lane) {
  using Sh = typename ST::Shift;
  constexpr int S = (int)sizeof(typename ST::Ring::E);
  using E = typename Elem<S>::E;
#pragma unroll
  for (int it = 0; it < Sh::SIT; ++it) {
    int c, q;
    lane_map<Sh::NCO, true>(it * Sh::NW + wave, lane, c, q);
    if (INNER || c < cols_left) {
      char *row_out = out + (c0 + c) * ld_out * S;
      const int d = (int)(((uintptr_t)row_out & 127) / S);
      const int64_t first = r0 - d + ST::V * q;
      typename ST::U w[ST::V];
#pragma unroll
      for (int k = 0; k < ST::V; ++k)
        w[k] = lds[ST::Ring::lds_index(ST::ring_row(first + k), c)];
      const u32x4 o = units_to_vec<S>(w);
      if (INNER || (first >= 0 && first + ST::V - 1 < rows)) {
        store16<CP>(row_out + first * S, o);
      } else {
        E e[ST::V];
        __builtin_memcpy(e, &o, 16);
#pragma unroll
        for (int x = 0; x < ST::V; ++x)
          if (first + x >= 0 && first + x < rows)
            reinterpret_cast<E *>(row_out)[first + x] = e[x];
      }
    }
  }
}

template <int S, int TR, int TC, int NT, int CP>
__global__ __launch_bounds__(NT) void xpose_shift_strip_kernel(TileArgs a,
                                                               uint32_t seg,
                                                               uint32_t nseg) {
  using ST = StripTile<S, TR, TC, NT, CP>;
  __shared__ __attribute__((aligned(16))) typename ST::U lds[ST::Ring::LDS_UNITS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t g = blockIdx.x;
  if (a.xcd_remap) {
    const uint32_t q = gridDim.x / 8, r = gridDim.x % 8, x = g % 8;
    g = x * q + (x < r ? x : r) + g / 8;
  }
  // Workgroups of one segment row are consecutive: neighbouring strips,
  // which share the input lines that straddle their column edge, run
  // together on one XCD.
  const uint32_t per = nseg * a.tiles_c;
  const int64_t b = (int64_t)(g / per) + a.batch_first;
  g %= per;
  const uint32_t tc = g % a.tiles_c, tr_first = (g / a.tiles_c) * seg;
  const uint32_t tr_end =
      tr_first + seg < a.tiles_r ? tr_first + seg : a.tiles_r;
  const int64_t c0 = (int64_t)tc * TC, cols_left = a.cols - c0;
  const char *in = static_cast<const char *>(a.in) + b * a.stride_in * S;
  char *out = static_cast<char *>(a.out) + b * a.stride_out * S;

  {  // the first tile's rows, its halo included
    const int64_t r0 = (int64_t)tr_first * TR;
    u32x4 h[ST::LIT_HALO];
    strip_load_any<ST>(h, in, r0 - ST::HALO, a.rows, a.ld_in, c0, cols_left,
                       wave, lane);
    strip_to_ring<ST>(lds, h, r0 - ST::HALO, wave, lane);
    u32x4 v[ST::LIT_NEW];
    strip_load_any<ST>(v, in, r0, a.rows, a.ld_in, c0, cols_left, wave, lane);
    strip_to_ring<ST>(lds, v, r0, wave, lane);
  }
  __syncthreads();
  // tr_first and tr_end are uniform per workgroup, so every wave takes the
  // same trips and reaches the same barriers.
  for (uint32_t tr = tr_first; tr < tr_end; ++tr) {
    const int64_t r0 = (int64_t)tr * TR;
    const bool more = tr + 1 < tr_end;
    u32x4 v[ST::LIT_NEW];
    if (more)
      strip_load_any<ST>(v, in, r0 + TR, a.rows, a.ld_in, c0, cols_left,
                         wave, lane);
    // Output row j = c0 + c, line-aligned segment from input row r0 - d_j
    // (as the one-shot line-aligned tile), its rows read from the ring.
    if (r0 >= ST::HALO && r0 + TR <= a.rows && cols_left >= TC)
      strip_store<ST, CP, true>(lds, out, r0, a.rows, a.ld_out, c0, cols_left,
                                wave, lane);
    else
      strip_store<ST, CP, false>(lds, out, r0, a.rows, a.ld_out, c0,
                                 cols_left, wave, lane);
    if (more) {
      __syncthreads();
      strip_to_ring<ST>(lds, v, r0 + TR, wave, lane);
      __syncthreads();
    }
  }
}

template <int S, int TR, int TC, int NT, int CP>
hipError_t launch_strip(const TileArgs &a, uint32_t seg, uint32_t nseg,
                        uint32_t grid, hipStream_t stream) {
  TileArgs copy = a;
  uint32_t sg = seg, ns = nseg;
  void *args[] = {&copy, &sg, &ns};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          &xpose_shift_strip_kernel<S, TR, TC, NT, CP>),
      dim3(grid), dim3(NT), args, 0, stream);
}

// ---------------------------------------------------------------------------
// Transpose-read tiles (1- and 2-byte elements).  gfx950's LDS transpose
// reads turn small blocks around on the way out of LDS.  Within each 16-lane
// group, with HR = 8 / S elements per 8 bytes and NQ = 16 / HR:
//   ds_read_b64_tr_b16 / _b8 give lane i, as its element m (m < HR),
//   element i % HR of the 8 bytes addressed by lane NQ * m + i / HR.
// (Checked on the hardware with distinct values at every address.)  So if
// lane NQ * m + q addresses 8-byte column unit cu of tile row R(q) + m, lane
// i receives column cu * HR + i % HR of rows R(i / HR) .. R(i / HR) + HR - 1.
// Two such reads give one 16-byte output vector of V = 2 HR rows.
//
// The LDS tile holds the input rows unchanged (no in-register packing).
// One group covers the HR columns of one 8-byte unit over 32 rows (NQ
// vectors per column); the four groups of a wave take four consecutive
// 32-row blocks of the same unit, so one store instruction writes up to 128
// consecutive rows of each of its HR output rows: whole 128-byte lines once
// TR >= 64 (2-byte elements) or 128 (1-byte).
//
// Banks: one read of a half-wave touches the same 8-byte unit of 32 rows,
// 256 bytes, which the 64 banks serve in one pass only if the 32 rows sit in
// 32 different 8-byte slots.  The rows differ in bits 0..5 except bit
// log2(HR); rows that the 256-byte window already separates by their row
// offset need nothing, the remaining varying bits XOR the 8-byte unit
// index.  A 16-byte chunk then keeps its two halves together, swapped when
// the mask is odd, so the row writes stay one ds_write_b128 per chunk.
// Direct global->LDS loads cannot swap halves: there the mask's lowest bit
// is dropped and the reads are 2-way conflicted.
// ---------------------------------------------------------------------------

// One transpose read at byte offset `off` (the address this lane supplies
// to its group).
template <int S>
__device__ __forceinline__ u32x2 tr_read(const uint8_t *lds, int off) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef int v2i32 __attribute__((ext_vector_type(2)));
  auto *p = (__attribute__((address_space(3))) uint8_t *)(lds + off);
  if constexpr (S == 2) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)p);
    return __builtin_bit_cast(u32x2, r);
  } else {
    const v2i32 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i32 *)p);
    return __builtin_bit_cast(u32x2, r);
  }
}

template <class T>
__device__ __forceinline__ void tr_write_chunk(uint8_t *lds, int row, int ch,
                                               u32x4 w) {
  int off;
  bool swap;
  T::chunk_at(row, ch, off, swap);
  *reinterpret_cast<u32x4 *>(lds + off) = swap ? u32x4{w.z, w.w, w.x, w.y} : w;
}

template <int S, int TR, int TC, int NT, int CP, bool DIRECT>
__global__ __launch_bounds__(NT) void xpose_tr_kernel(TileArgs a) {
  using T = TrTile<S, TR, TC, NT, CP, DIRECT>;
  using E = typename Elem<S>::E;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const TileSpot p = tile_spot<S, TR, TC>(a, blockIdx.x, gridDim.x);
  constexpr int RPT = 64 / T::NCL;  // tile rows per wave load task

  // Phase 1: rows of the tile into LDS, 16 bytes per lane.
  if (p.vec) {
    if constexpr (DIRECT) {
      // Lane l fills physical slot l of the wave's 1 KiB: it fetches the
      // logical chunk that the (even) mask puts there.
#pragma unroll
      for (int it = 0; it < T::LIT; ++it) {
        const int wt = it * T::NW + wave;
        const int row = wt * RPT + lane / T::NCL;
        const int chunk = (lane % T::NCL) ^ (T::swz(row) >> 1);
        __builtin_amdgcn_global_load_lds(
            p.src + (int64_t)row * a.ld_in * S + chunk * 16,
            (__attribute__((address_space(3))) void *)(lds + wt * 1024), 16,
            0, 0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      u32x4 v[T::LIT];
#pragma unroll
      for (int it = 0; it < T::LIT; ++it) {
        const int row = (it * T::NW + wave) * RPT + lane / T::NCL;
        v[it] = load16<CP == kNtLoadStore ? kNtLoadStore : kCacheDefault>(
            p.src + (int64_t)row * a.ld_in * S + (lane % T::NCL) * 16);
      }
#pragma unroll
      for (int it = 0; it < T::LIT; ++it) {
        const int row = (it * T::NW + wave) * RPT + lane / T::NCL;
        tr_write_chunk<T>(lds, row, lane % T::NCL, v[it]);
      }
    }
  } else {
    // Edge tile: whole 16-byte chunks inside the matrix still move as one
    // access when the call allows it (a.vec_ok is uniform over the launch).
#pragma unroll
    for (int it = 0; it < T::LIT; ++it) {
      const int row = (it * T::NW + wave) * RPT + lane / T::NCL;
      const int ch = lane % T::NCL;
      const char *rs = p.src + ((int64_t)row * a.ld_in + ch * T::V) * S;
      u32x4 w;
      if (a.vec_ok && row < p.rows_left && (ch + 1) * T::V <= p.cols_left) {
        w = load16<CP == kNtLoadStore ? kNtLoadStore : kCacheDefault>(rs);
      } else {
        E e[T::V];
#pragma unroll
        for (int x = 0; x < T::V; ++x)
          e[x] = (row < p.rows_left && ch * T::V + x < p.cols_left)
                     ? reinterpret_cast<const E *>(rs)[x]
                     : E(0);
        __builtin_memcpy(&w, e, 16);
      }
      tr_write_chunk<T>(lds, row, ch, w);
    }
  }
  __syncthreads();

  // Phase 2: group q of the wave takes 32-row block rb of 8-byte column
  // unit cu; the four groups of a wave take consecutive row blocks.
  const int q = lane >> 4, i = lane & 15;
#pragma unroll
  for (int it = 0; it < T::SIT; ++it) {
    const int gt = (it * T::NW + wave) * 4 + q;
    const int rb = gt % T::NRB, cu = gt / T::NRB;
    u32x2 h[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = rb * 32 + (i % T::NQ) * T::V + k * T::HR + i / T::NQ;
      h[k] = tr_read<S>(lds, T::unit_at(row, cu));
    }
    const u32x4 o = u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
    const int c = cu * T::HR + i % T::HR;       // output row in the tile
    const int r = rb * 32 + (i / T::HR) * T::V;  // first input row
    char *dst = p.dst + ((int64_t)c * a.ld_out + r) * S;
    if (p.vec || (a.vec_ok && c < p.cols_left && r + T::V <= p.rows_left)) {
      store16<CP>(dst, o);
    } else if (c < p.cols_left) {
      E e[T::V];
      __builtin_memcpy(e, &o, 16);
#pragma unroll
      for (int x = 0; x < T::V; ++x)
        if (r + x < p.rows_left) reinterpret_cast<E *>(dst)[x] = e[x];
    }
  }
}

template <int S, int TR, int TC, int NT, int CP, bool DIRECT>
hipError_t launch_tr(const TileArgs &a, uint32_t grid, uint32_t lds_extra,
                     hipStream_t stream) {
  TileArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(&xpose_tr_kernel<S, TR, TC, NT, CP, DIRECT>),
      dim3(grid), dim3(NT), args, lds_extra, stream);
}

#define XPOSE_TR(S, TR, TC, NT, CP, D)                                      \
  TileKernel {                                                              \
    S, TR, TC, NT, kSwizzle, CP, TrTile<S, TR, TC, NT, CP, D>::LDS_BYTES,  \
        &launch_tr<S, TR, TC, NT, CP, D>, nullptr, D, false, true           \
  }

#define XPOSE_SHIFT(S, TR, TC, NT, CP)                                      \
  TileKernel {                                                              \
    S, TR, TC, NT, kSwizzle, CP, ShiftTile<S, TR, TC, NT, CP>::LDS_BYTES,  \
        &launch_shift<S, TR, TC, NT, CP>, nullptr, false, true              \
  }
// Also built as column strips (4- and 8-byte elements).
#define XPOSE_SHIFT_S(S, TR, TC, NT, CP)                                    \
  TileKernel {                                                              \
    S, TR, TC, NT, kSwizzle, CP, ShiftTile<S, TR, TC, NT, CP>::LDS_BYTES,  \
        &launch_shift<S, TR, TC, NT, CP>, nullptr, false, true, false,      \
        &launch_strip<S, TR, TC, NT, CP>,                                   \
        StripTile<S, TR, TC, NT, CP>::LDS_BYTES                             \
  }

#define XPOSE_TILE(S, TR, TC, NT, L, CP)                                    \
  TileKernel {                                                              \
    S, TR, TC, NT, L, CP, Tile<S, TR, TC, NT, L, CP>::LDS_BYTES,           \
        &launch_tile<S, TR, TC, NT, L, CP>, nullptr, false, false           \
  }
// Interior tiles loaded straight into LDS.
#define XPOSE_TILE_D(S, TR, TC, NT, L, CP)                                  \
  TileKernel {                                                              \
    S, TR, TC, NT, L, CP, Tile<S, TR, TC, NT, L, CP, true>::LDS_BYTES,     \
        &launch_tile<S, TR, TC, NT, L, CP, true>, nullptr, true, false      \
  }
// Also built as a persistent, double-buffered kernel.
#define XPOSE_TILE_P(S, TR, TC, NT, L, CP)                                  \
  TileKernel {                                                              \
    S, TR, TC, NT, L, CP, Tile<S, TR, TC, NT, L, CP>::LDS_BYTES,           \
        &launch_tile<S, TR, TC, NT, L, CP>,                                 \
        &launch_tile_persistent<S, TR, TC, NT, L, CP>, false, false         \
  }
// Every layout with plain caching and with non-temporal stores (so the
// layout ablation compares like with like).
#define XPOSE_TILES(S, TR, TC, NT)                                          \
  XPOSE_TILE_P(S, TR, TC, NT, kSwizzle, kCacheDefault),                     \
      XPOSE_TILE(S, TR, TC, NT, kPad1, kCacheDefault),                      \
      XPOSE_TILE(S, TR, TC, NT, kUnpadded, kCacheDefault),                  \
      XPOSE_TILE_P(S, TR, TC, NT, kSwizzle, kNtStore),                      \
      XPOSE_TILE(S, TR, TC, NT, kPad1, kNtStore),                           \
      XPOSE_TILE(S, TR, TC, NT, kUnpadded, kNtStore)

// Every layout and both cache policies, one LDS buffer only (tiles whose
// double-buffered persistent kernel would not fit the LDS).
#define XPOSE_TILES_1(S, TR, TC, NT)                                        \
  XPOSE_TILE(S, TR, TC, NT, kSwizzle, kCacheDefault),                       \
      XPOSE_TILE(S, TR, TC, NT, kPad1, kCacheDefault),                      \
      XPOSE_TILE(S, TR, TC, NT, kUnpadded, kCacheDefault),                  \
      XPOSE_TILE(S, TR, TC, NT, kSwizzle, kNtStore),                        \
      XPOSE_TILE(S, TR, TC, NT, kPad1, kNtStore),                           \
      XPOSE_TILE(S, TR, TC, NT, kUnpadded, kNtStore)

static const TileKernel kTileKernels[] = {
    // 4-byte elements
    XPOSE_TILES(4, 32, 32, 256), XPOSE_TILES(4, 32, 32, 128),
    XPOSE_TILES(4, 32, 32, 64), XPOSE_TILES(4, 32, 64, 128),
    XPOSE_TILES(4, 64, 32, 128), XPOSE_TILES(4, 64, 64, 256),
    XPOSE_TILES(4, 64, 128, 256), XPOSE_TILES(4, 128, 64, 256),
    XPOSE_TILES(4, 128, 128, 256), XPOSE_TILES(4, 32, 128, 256),
    XPOSE_TILES(4, 128, 32, 256),
    XPOSE_TILES_1(4, 256, 128, 256),
    XPOSE_TILE(4, 32, 32, 256, kSwizzle, kNtLoadStore),
    XPOSE_TILE_D(4, 32, 32, 256, kSwizzle, kNtStore),
    XPOSE_TILE_D(4, 32, 32, 256, kSwizzle, kCacheDefault),
    XPOSE_TILE_D(4, 32, 32, 256, kUnpadded, kNtStore),
    XPOSE_TILE_D(4, 64, 64, 256, kSwizzle, kNtStore),
    XPOSE_TILE_D(4, 64, 64, 256, kSwizzle, kCacheDefault),
    XPOSE_TILE_D(4, 128, 64, 256, kSwizzle, kNtStore),
    XPOSE_TILE_D(4, 128, 64, 256, kSwizzle, kCacheDefault),
    XPOSE_TILE_D(8, 32, 32, 256, kSwizzle, kNtStore),
    XPOSE_TILE_D(8, 32, 32, 256, kSwizzle, kCacheDefault),
    // Line-aligned output tiles (4-byte elements).
    XPOSE_SHIFT_S(4, 64, 64, 256, kNtStore),
    XPOSE_SHIFT(4, 64, 64, 256, kCacheDefault),
    XPOSE_SHIFT_S(4, 128, 64, 256, kNtStore),
    XPOSE_SHIFT(4, 128, 64, 256, kCacheDefault),
    XPOSE_SHIFT(4, 256, 64, 256, kNtStore),
    XPOSE_SHIFT(4, 256, 64, 256, kCacheDefault),
    XPOSE_SHIFT_S(4, 128, 32, 256, kNtStore), XPOSE_SHIFT(4, 64, 32, 128, kNtStore),
    XPOSE_SHIFT(4, 64, 128, 256, kNtStore),
    XPOSE_SHIFT(4, 128, 128, 256, kNtStore),
    XPOSE_SHIFT(4, 256, 128, 256, kNtStore),
    XPOSE_TILE(4, 64, 64, 256, kSwizzle, kNtLoadStore),
    // 2-byte elements
    XPOSE_TILES(2, 32, 32, 64), XPOSE_TILES(2, 32, 64, 128),
    XPOSE_TILES(2, 64, 32, 128), XPOSE_TILES(2, 64, 64, 128),
    XPOSE_TILES(2, 64, 64, 256), XPOSE_TILES(2, 128, 128, 256),
    XPOSE_TILES(2, 64, 128, 256), XPOSE_TILES(2, 128, 64, 256),
    XPOSE_TILES_1(2, 256, 256, 256), XPOSE_TILES_1(2, 256, 256, 512),
    // Line-aligned output tiles (2-byte elements).
    XPOSE_SHIFT(2, 64, 64, 256, kNtStore),
    XPOSE_SHIFT(2, 64, 64, 256, kCacheDefault),
    XPOSE_SHIFT(2, 128, 64, 256, kNtStore),
    XPOSE_SHIFT(2, 128, 64, 256, kCacheDefault),
    XPOSE_SHIFT(2, 256, 64, 256, kNtStore),
    // 2-byte elements through LDS transpose reads
    XPOSE_TR(2, 64, 64, 256, kNtStore, false),
    XPOSE_TR(2, 64, 64, 256, kCacheDefault, false),
    XPOSE_TR(2, 128, 64, 256, kNtStore, false),
    XPOSE_TR(2, 128, 64, 256, kCacheDefault, false),
    XPOSE_TR(2, 64, 128, 256, kNtStore, false),
    XPOSE_TR(2, 64, 128, 256, kCacheDefault, false),
    XPOSE_TR(2, 128, 128, 256, kNtStore, false),
    XPOSE_TR(2, 128, 128, 256, kCacheDefault, false),
    XPOSE_TR(2, 64, 32, 128, kNtStore, false),
    XPOSE_TR(2, 64, 64, 256, kNtStore, true),
    XPOSE_TR(2, 64, 64, 256, kCacheDefault, true),
    XPOSE_TR(2, 128, 64, 256, kNtStore, true),
    XPOSE_TR(2, 128, 64, 256, kCacheDefault, true),
    XPOSE_TR(2, 128, 128, 256, kNtStore, true),
    // 1-byte elements
    XPOSE_TILES(1, 64, 64, 64), XPOSE_TILES(1, 64, 128, 128),
    XPOSE_TILES(1, 128, 64, 128), XPOSE_TILES(1, 128, 128, 256),
    XPOSE_TR(1, 128, 128, 256, kNtStore, false),
    XPOSE_TR(1, 128, 128, 256, kCacheDefault, false),
    XPOSE_TR(1, 64, 128, 128, kNtStore, false),
    XPOSE_TR(1, 128, 64, 128, kNtStore, false),
    XPOSE_TR(1, 128, 256, 256, kNtStore, false),
    XPOSE_TR(1, 128, 128, 256, kNtStore, true),
    XPOSE_TR(1, 128, 128, 256, kCacheDefault, true),
    // 8-byte elements
    XPOSE_TILES(8, 32, 32, 128),
    XPOSE_TILES(8, 32, 32, 256), XPOSE_TILES(8, 64, 64, 256),
    XPOSE_TILES_1(8, 128, 128, 256),
    // Line-aligned output tiles (8-byte elements).
    XPOSE_SHIFT_S(8, 32, 32, 256, kNtStore),
    XPOSE_SHIFT(8, 32, 32, 256, kCacheDefault),
    XPOSE_SHIFT_S(8, 64, 32, 256, kNtStore),
    XPOSE_SHIFT(8, 64, 64, 256, kNtStore),
    XPOSE_SHIFT(8, 64, 64, 256, kCacheDefault),
};

const TileKernel *tile_kernels(int *count) {
  *count = (int)(sizeof(kTileKernels) / sizeof(kTileKernels[0]));
  return kTileKernels;
}

// ---------------------------------------------------------------------------
// Packed batches of small matrices.  A batch of dense small matrices (row
// length = pitch, matrix stride = rows * cols) is one contiguous array on
// each side, and a whole number of matrices is one contiguous range on each
// side.  So a workgroup takes per_block whole matrices: it reads their bytes
// with 16-byte loads into LDS, waits at the barrier, and writes the same
// number of output bytes with 16-byte stores, each lane gathering the V
// elements of its output vector from LDS.  Where the ordinary tile would be
// mostly empty (a 16 x 16 fp32 matrix fills 1/32 of a 128 x 64 tile), this
// keeps every global access whole and every lane busy.
// ---------------------------------------------------------------------------
// LDS padding.  Where input rows are a multiple of 64 bytes the output
// vectors of a half-wave, which step down input columns, would fall on a few
// banks; a pad of one 4-byte word (8 bytes for 8-byte elements) after every
// input row makes the row stride odd in words.  Rows then start 4-byte but
// not 16-byte aligned in LDS, so the padded block is written in 32-bit
// words.  The pad adds at most 1/8 to the block.
template <int S, int NT, int BB, int CP>
__global__ __launch_bounds__(NT) void xpose_packed_kernel(PackedArgs a) {
  using E = typename Elem<S>::E;
  constexpr int V = 16 / S;
  __shared__ __attribute__((aligned(16))) E lds[(BB + BB / 8) / S];
  const uint32_t rows = a.rows, cols = a.cols, m = rows * cols, pad = a.pad;
  const uint32_t cs = cols + pad, mp = rows * cs;  // padded strides
  const int64_t m0 = (int64_t)blockIdx.x * a.per_block;  // first matrix
  const int64_t left = a.count - m0;
  const uint32_t nmat = left < a.per_block ? (uint32_t)left : a.per_block;
  const uint32_t n = nmat * m;  // elements of this workgroup
  const char *src = static_cast<const char *>(a.in) + m0 * m * S;
  char *dst = static_cast<char *>(a.out) + m0 * m * S;
  const uint32_t nv = n / V;  // whole 16-byte vectors

  // Phase 1: the block's input bytes, in order, into LDS.  Every lane
  // issues its NIT loads before the first LDS write: lanes past the block's
  // last vector reload that vector (in bounds, same line) instead of
  // branching around the load, which would make the compiler wait for each
  // load before issuing the next.
  constexpr int NIT = (BB / 16 + NT - 1) / NT;
  constexpr int LCP = CP == kNtLoadStore ? kNtLoadStore : kCacheDefault;
  if (nv > 0) {  // uniform per workgroup
    u32x4 w[NIT];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const uint32_t v = threadIdx.x + k * NT;
      w[k] = load16<LCP>(src + (v < nv ? v : nv - 1) * 16);
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const uint32_t v = threadIdx.x + k * NT;
      if (v >= nv) continue;
      const uint32_t e = v * V;
      if (pad == 0) {
        *reinterpret_cast<u32x4 *>(lds + e) = w[k];
      } else {
        // Rows are whole 16-byte vectors here (cols * S is a multiple of
        // 64), so a vector never crosses a padded row end.
        uint32_t *d = reinterpret_cast<uint32_t *>(lds + e + e / cols * pad);
        d[0] = w[k].x;
        d[1] = w[k].y;
        d[2] = w[k].z;
        d[3] = w[k].w;
      }
    }
  }
  if (pad == 0)
    for (uint32_t e = nv * V + threadIdx.x; e < n; e += NT)
      lds[e] = reinterpret_cast<const E *>(src)[e];
  __syncthreads();

  // Phase 2: output element o of the block is element (j, i) of output
  // matrix g (o = g m + j rows + i), which is input element g m + i cols + j,
  // at LDS element g mp + i cs + j.  The V elements of one vector step down
  // an input column (stride cs); where the vector runs past the column's
  // last row it continues at the next column's first row, and past the last
  // column at the next matrix.
  for (uint32_t v = threadIdx.x; v < nv; v += NT) {
    const uint32_t o = v * V, g = o / m, t = o - g * m;
    uint32_t j = t / rows, i = t - j * rows;
    uint32_t at = g * mp + i * cs + j;  // unsigned wrap-around is intended
    E e[V];
    if (i + V <= rows) {
#pragma unroll
      for (int x = 0; x < V; ++x) e[x] = lds[at + x * cs];
    } else {
#pragma unroll
      for (int x = 0; x < V; ++x) {
        e[x] = lds[at];
        at += cs;
        if (++i == rows) {  // row past the column: next column, row 0
          i = 0;
          at += 1 - mp;
          if (++j == cols) {  // past the last column: next matrix
            j = 0;
            at += mp - cols;
          }
        }
      }
    }
    u32x4 w;
    __builtin_memcpy(&w, e, 16);
    store16<CP>(dst + v * 16, w);
  }
  for (uint32_t o = nv * V + threadIdx.x; o < n; o += NT) {
    const uint32_t g = o / m, t = o - g * m, j = t / rows, i = t - j * rows;
    reinterpret_cast<E *>(dst)[o] = lds[g * mp + i * cs + j];
  }
}

template <int S, int NT, int BB, int CP>
hipError_t launch_packed(const PackedArgs &a, uint32_t grid,
                         hipStream_t stream) {
  PackedArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(&xpose_packed_kernel<S, NT, BB, CP>),
      dim3(grid), dim3(NT), args, 0, stream);
}

#define XPOSE_PACKED(S, BB, CP) \
  PackedKernel { S, 256, BB, CP, &launch_packed<S, 256, BB, CP> }
#define XPOSE_PACKED_ALL(BB)                                               \
  XPOSE_PACKED(1, BB, kNtStore), XPOSE_PACKED(1, BB, kCacheDefault),       \
      XPOSE_PACKED(2, BB, kNtStore), XPOSE_PACKED(2, BB, kCacheDefault),   \
      XPOSE_PACKED(4, BB, kNtStore), XPOSE_PACKED(4, BB, kCacheDefault),   \
      XPOSE_PACKED(8, BB, kNtStore), XPOSE_PACKED(8, BB, kCacheDefault)

// Smaller blocks first: the planner takes the first block size in which a
// whole number of matrices makes whole cache lines.
static const PackedKernel kPackedKernels[] = {XPOSE_PACKED_ALL(16384),
                                              XPOSE_PACKED_ALL(32768)};

const PackedKernel *packed_kernels(int *count) {
  *count = (int)(sizeof(kPackedKernels) / sizeof(kPackedKernels[0]));
  return kPackedKernels;
}

// ---------------------------------------------------------------------------
// Naive single-index transposes, the ablation baseline without LDS: one
// element per thread.  Read-coalesced blocks run along an input row (the
// reads are contiguous, each write lands one output row further on);
// write-coalesced blocks run along an input column (contiguous writes,
// strided reads).  Either way one of the two global sides is uncoalesced,
// which is the cost the LDS tile removes ("Shared memory and the bank
// conflict", section "Turn the tile around on chip").
//   grid.x: 256-element runs along the coalesced side; grid.y: index along
//   the other side (offset by `other0`); grid.z: batch entry (offset by
//   a.batch_first).
// ---------------------------------------------------------------------------
constexpr int kNaiveThreads = 256;

template <int S, bool READ_COALESCED>
__global__ __launch_bounds__(kNaiveThreads) void xpose_naive_kernel(
    TileArgs a, int64_t other0) {
  using E = typename Elem<S>::E;
  const int64_t run = (int64_t)blockIdx.x * kNaiveThreads + threadIdx.x;
  const int64_t other = other0 + blockIdx.y;
  const int64_t b = (int64_t)blockIdx.z + a.batch_first;
  const int64_t i = READ_COALESCED ? other : run;  // input row
  const int64_t j = READ_COALESCED ? run : other;  // input column
  if (i >= a.rows || j >= a.cols) return;
  const E v = static_cast<const E *>(a.in)[b * a.stride_in + i * a.ld_in + j];
  static_cast<E *>(a.out)[b * a.stride_out + j * a.ld_out + i] = v;
}

template <int S, bool RC>
hipError_t launch_naive_s(const TileArgs &a, int64_t batch,
                          hipStream_t stream) {
  const int64_t run_len = RC ? a.cols : a.rows;
  const int64_t others = RC ? a.rows : a.cols;
  const int64_t gx = (run_len + kNaiveThreads - 1) / kNaiveThreads;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  for (int64_t b0 = 0; b0 < batch; b0 += 65535) {
    for (int64_t o0 = 0; o0 < others; o0 += 65535) {
      TileArgs c = a;
      c.batch_first = (uint32_t)0;
      c.in = static_cast<const char *>(a.in) + b0 * a.stride_in * S;
      c.out = static_cast<char *>(a.out) + b0 * a.stride_out * S;
      int64_t off = o0;
      const dim3 grid((uint32_t)gx,
                      (uint32_t)(others - o0 < 65535 ? others - o0 : 65535),
                      (uint32_t)(batch - b0 < 65535 ? batch - b0 : 65535));
      void *args[] = {&c, &off};
      const hipError_t e = hipLaunchKernel(
          reinterpret_cast<const void *>(&xpose_naive_kernel<S, RC>), grid,
          dim3(kNaiveThreads), args, 0, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_naive(const TileArgs &a, int64_t batch, int elem_bytes,
                        bool read_coalesced, hipStream_t stream) {
  switch (elem_bytes) {
    case 1: return read_coalesced ? launch_naive_s<1, true>(a, batch, stream)
                                  : launch_naive_s<1, false>(a, batch, stream);
    case 2: return read_coalesced ? launch_naive_s<2, true>(a, batch, stream)
                                  : launch_naive_s<2, false>(a, batch, stream);
    case 4: return read_coalesced ? launch_naive_s<4, true>(a, batch, stream)
                                  : launch_naive_s<4, false>(a, batch, stream);
    case 8: return read_coalesced ? launch_naive_s<8, true>(a, batch, stream)
                                  : launch_naive_s<8, false>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Copy yardstick.  Each workgroup moves NT * UNROLL 16-byte vectors of one
// contiguous range, issuing all its loads before its stores, exactly the
// access widths the transpose uses.  The default (256 threads x 4) moves the
// same 16 KiB in and out per workgroup as a 64 x 64 fp32 tile.
// ---------------------------------------------------------------------------
template <int NT, int UNROLL, int CP>
__global__ __launch_bounds__(NT) void copy16_kernel(char *__restrict__ dst,
                                                    const char *__restrict__ src,
                                                    int64_t nvec) {
  const int64_t base = (int64_t)blockIdx.x * (NT * UNROLL) + threadIdx.x;
  u32x4 r[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = base + (int64_t)u * NT;
    if (i < nvec) r[u] = load16<CP>(src + i * 16);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = base + (int64_t)u * NT;
    if (i < nvec) store16<CP>(dst + i * 16, r[u]);
  }
}

__global__ __launch_bounds__(256) void copy_bytes_kernel(
    char *__restrict__ dst, const char *__restrict__ src, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += step)
    dst[i] = src[i];
}

template <int NT, int UNROLL, int CP>
hipError_t launch_copy16(char *d, const char *s, int64_t nvec,
                         hipStream_t stream) {
  const int64_t per_block = (int64_t)NT * UNROLL;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void *args[] = {&d, &s, &nvec};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(&copy16_kernel<NT, UNROLL, CP>),
      dim3((uint32_t)blocks), dim3(NT), args, 0, stream);
}

#define XPOSE_COPY(NT, U, CP) CopyKernel{NT, U, CP, &launch_copy16<NT, U, CP>}
static const CopyKernel kCopyKernels[] = {
    XPOSE_COPY(256, 1, kCacheDefault), XPOSE_COPY(256, 2, kCacheDefault),
    XPOSE_COPY(256, 4, kCacheDefault), XPOSE_COPY(256, 8, kCacheDefault),
    XPOSE_COPY(512, 4, kCacheDefault), XPOSE_COPY(1024, 4, kCacheDefault),
    XPOSE_COPY(64, 4, kNtStore),       XPOSE_COPY(128, 2, kNtStore),
    XPOSE_COPY(256, 1, kNtStore),      XPOSE_COPY(256, 2, kNtStore),
    XPOSE_COPY(256, 4, kNtStore),      XPOSE_COPY(256, 8, kNtStore),
    XPOSE_COPY(512, 1, kNtStore),      XPOSE_COPY(512, 2, kNtStore),
    XPOSE_COPY(1024, 1, kNtStore),     XPOSE_COPY(256, 1, kNtLoadStore),
    XPOSE_COPY(256, 4, kNtLoadStore),
};

const CopyKernel *copy_kernels(int *count) {
  *count = (int)(sizeof(kCopyKernels) / sizeof(kCopyKernels[0]));
  return kCopyKernels;
}

hipError_t launch_copy(const CopyKernel &k, void *dst, const void *src,
                       int64_t bytes, hipStream_t stream) {
  char *d = static_cast<char *>(dst);
  const char *s = static_cast<const char *>(src);
  int64_t head = 0;
  if ((((uintptr_t)d | (uintptr_t)s) & 15) == 0) {
    const int64_t nvec = bytes / 16;
    if (nvec > 0) {
      const hipError_t e = k.launch(d, s, nvec, stream);
      if (e != hipSuccess) return e;
    }
    head = nvec * 16;
  }
  int64_t rest = bytes - head;
  if (rest > 0) {
    char *dd = d + head;
    const char *ss = s + head;
    int64_t blocks = (rest + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *args[] = {&dd, &ss, &rest};
    return hipLaunchKernel(reinterpret_cast<const void *>(&copy_bytes_kernel),
                           dim3((uint32_t)blocks), dim3(256), args, 0, stream);
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// LDS bank microbenchmark.  One wavefront; lane l accesses byte offset
// lane_bytes[l] + k * 2048 (k = 0..7) of a 32 KiB LDS buffer with one LDS
// instruction per k.  2048 bytes is a multiple of any plausible bank period,
// so all eight instructions see the same bank pattern.  The instructions are
// written as inline assembly so the compiler can neither merge nor reorder
// them; no wait is placed between them inside the loop, so the elapsed time
// measures issue throughput, which an n-way conflict divides by n.
// ---------------------------------------------------------------------------
struct ProbeLanes {
  int32_t b[64];
};

#define PROBE_RD8(OP, T)                                                   \
  asm volatile(OP " %0, %8\n\t" OP " %1, %8 offset:2048\n\t" OP            \
                  " %2, %8 offset:4096\n\t" OP " %3, %8 offset:6144\n\t" OP  \
                  " %4, %8 offset:8192\n\t" OP " %5, %8 offset:10240\n\t" OP \
                  " %6, %8 offset:12288\n\t" OP " %7, %8 offset:14336"       \
               : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), \
                 "+v"(r6), "+v"(r7)                                          \
               : "v"(addr))
#define PROBE_WR8(OP)                                                        \
  asm volatile(OP " %0, %1\n\t" OP " %0, %1 offset:2048\n\t" OP              \
                  " %0, %1 offset:4096\n\t" OP " %0, %1 offset:6144\n\t" OP  \
                  " %0, %1 offset:8192\n\t" OP " %0, %1 offset:10240\n\t" OP \
                  " %0, %1 offset:12288\n\t" OP " %0, %1 offset:14336"       \
               :                                                             \
               : "v"(addr), "v"(r0)                                          \
               : "memory")

template <int W, bool WRITE>
__global__ __launch_bounds__(64) void lds_probe_kernel(ProbeLanes lanes,
                                                       int iters,
                                                       uint64_t *out) {
  using R = typename std::conditional<
      W == 4, uint32_t,
      typename std::conditional<W == 8, u32x2, u32x4>::type>::type;
  __shared__ __attribute__((aligned(16))) uint32_t buf[8192];
  const int lane = threadIdx.x;
  for (int i = lane; i < 8192; i += 64) buf[i] = (uint32_t)i * 0x9E3779B1u;
  __syncthreads();
  // LDS byte address of this lane's target: the buffer's own LDS offset
  // plus the lane's byte offset.
  const uint32_t base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint32_t *)buf);
  const uint32_t addr = base + (uint32_t)lanes.b[lane];
  R r0{}, r1{}, r2{}, r3{}, r4{}, r5{}, r6{}, r7{};
  if constexpr (WRITE) r0 = R{} + (uint32_t)lane;
  // Materialise the address (a kernel-argument load) before the clock starts.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : "v"(addr) : "memory");
  const uint64_t t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    if constexpr (WRITE) {
      if constexpr (W == 4) PROBE_WR8("ds_write_b32");
      else if constexpr (W == 8) PROBE_WR8("ds_write_b64");
      else PROBE_WR8("ds_write_b128");
    } else {
      if constexpr (W == 4) PROBE_RD8("ds_read_b32", R);
      else if constexpr (W == 8) PROBE_RD8("ds_read_b64", R);
      else PROBE_RD8("ds_read_b128", R);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint64_t t1 = clock64();
  R acc = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
  uint32_t sum;
  if constexpr (W == 4) sum = acc;
  else if constexpr (W == 8) sum = acc.x ^ acc.y;
  else sum = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (lane == 0) out[0] = t1 - t0;
  if (lane == 0) out[1] = sum;
}

hipError_t launch_lds_probe(uint64_t *out, const int32_t *lane_bytes,
                            int width, bool is_write, int iters,
                            hipStream_t stream) {
  ProbeLanes lanes;
  for (int i = 0; i < 64; ++i) lanes.b[i] = lane_bytes[i];
  const void *fn;
  if (width == 4)
    fn = is_write ? (const void *)&lds_probe_kernel<4, true>
                  : (const void *)&lds_probe_kernel<4, false>;
  else if (width == 8)
    fn = is_write ? (const void *)&lds_probe_kernel<8, true>
                  : (const void *)&lds_probe_kernel<8, false>;
  else
    fn = is_write ? (const void *)&lds_probe_kernel<16, true>
                  : (const void *)&lds_probe_kernel<16, false>;
  void *args[] = {&lanes, &iters, &out};
  return hipLaunchKernel(fn, dim3(1), dim3(64), args, 0, stream);
}

}  // namespace xpose
