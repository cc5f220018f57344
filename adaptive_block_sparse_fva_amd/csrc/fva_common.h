// Internal definitions shared by the libfva kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/fva.h"

namespace fva {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Division by a runtime constant d >= 1 for dividends n < 2^31, with a
// multiplier chosen on the host: q = (mulhi(n, m) + n) >> s, where
// s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
  __host__ __device__ FastDiv() : d(1), m(0), s(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    s = 0;
    while ((1ull << s) < div) ++s;
    m = (uint32_t)(((1ull << 32) * ((1ull << s) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, m) + n) >> s;
  }
};

// Geometry of the video-aware order: frames of grid_h x grid_w tokens split
// into tile_h x tile_w spatial tiles (raster order of tiles, raster inside a
// tile, tiles cut at the frame border).  Position -> natural token index.
struct OrderGeo {
  int32_t kind;                // FVA_ORDER_TILES or FVA_ORDER_HILBERT
  int32_t n, hw, gw, th, tw;   // tokens, grid_h*grid_w, grid_w, tile dims (0 = raster)
  int32_t gh;                  // grid_h
  FastDiv div_hw;              // by grid_h*grid_w
  FastDiv div_band;            // by tile_h*grid_w (a full band of tile rows)
  FastDiv div_tile_full;       // by tile_h*tile_w (tile in a full band)
  FastDiv div_tile_last;       // by last_h*tile_w (tile in the short last band)
  FastDiv div_w_full;          // by tile_w
  FastDiv div_w_last;          // by last_w (short last tile column)
  int32_t last_h, last_w;      // height of the last band, width of the last tile column

  // Cell d of a frame along the generalised Hilbert curve (the walk the
  // header describes), found by descending its recursion: at each level the
  // part holding d, with the part's origin and axes.
  __device__ __forceinline__ int32_t hilbert_cell(int32_t d) const {
    int32_t ox = 0, oy = 0, ax = 1, ay = 0, bx = 0, by = 1, w = gw, h = gh;
    for (;;) {
      if (h == 1) { ox += d * ax; oy += d * ay; break; }
      if (w == 1) { ox += d * bx; oy += d * by; break; }
      const int32_t w0 = (w + 1) >> 1;
      if (w > 2 * h) {
        if (d < w0 * h) {
          w = w0;
        } else {
          d -= w0 * h;
          ox += w0 * ax; oy += w0 * ay;
          w -= w0;
        }
        continue;
      }
      int32_t t0;
      if (h > 2 * w) {
        if (d < h * w0) {
          t0 = ax; ax = bx; bx = t0;
          t0 = ay; ay = by; by = t0;
          const int32_t nw = h; h = w0; w = nw;
        } else {
          d -= h * w0;
          ox += (w - 1) * ax + (h - 1) * bx; oy += (w - 1) * ay + (h - 1) * by;
          t0 = ax; ax = -bx; bx = -t0;
          t0 = ay; ay = -by; by = -t0;
          const int32_t nw = h; h = w - w0; w = nw;
        }
        continue;
      }
      const int32_t h0 = (h + 1) >> 1, w1 = w - w0, h1 = h - h0;
      const int32_t s0 = h0 * w0, s1 = w0 * h1, s2 = w1 * h1;
      if (d < s0) {
        t0 = ax; ax = bx; bx = t0;
        t0 = ay; ay = by; by = t0;
        w = h0; h = w0;
      } else if (d < s0 + s1) {
        d -= s0;
        ox += h0 * bx; oy += h0 * by;
        w = w0; h = h1;
      } else if (d < s0 + s1 + s2) {
        d -= s0 + s1;
        ox += h0 * bx + w0 * ax; oy += h0 * by + w0 * ay;
        w = w1; h = h1;
      } else {
        d -= s0 + s1 + s2;
        ox += (w - 1) * ax + (h0 - 1) * bx; oy += (w - 1) * ay + (h0 - 1) * by;
        t0 = ax; ax = -bx; bx = -t0;
        t0 = ay; ay = -by; by = -t0;
        w = h0; h = w1;
      }
    }
    return oy * gw + ox;
  }

  __device__ __forceinline__ int32_t token(int32_t pos) const {
    if (pos >= n) return -1;
    if (kind == FVA_ORDER_HILBERT) {
      const uint32_t t = div_hw.div((uint32_t)pos);
      return (int32_t)(t * (uint32_t)hw) + hilbert_cell(pos - (int32_t)(t * (uint32_t)hw));
    }
    if (th == 0) return pos;
    const uint32_t t = div_hw.div((uint32_t)pos);
    const uint32_t r = (uint32_t)pos - t * (uint32_t)hw;
    const uint32_t band = div_band.div(r);
    const uint32_t r2 = r - band * (uint32_t)(th * gw);
    const bool last_band = (int32_t)(band + 1) * th > gh;
    const uint32_t bh = last_band ? (uint32_t)last_h : (uint32_t)th;
    const uint32_t ct = last_band ? div_tile_last.div(r2) : div_tile_full.div(r2);
    const uint32_t r3 = r2 - ct * bh * (uint32_t)tw;
    const bool last_col = (int32_t)(ct + 1) * tw > gw;
    const uint32_t y = last_col ? div_w_last.div(r3) : div_w_full.div(r3);
    const uint32_t w = last_col ? (uint32_t)last_w : (uint32_t)tw;
    const uint32_t x = r3 - y * w;
    return (int32_t)(t * (uint32_t)hw + (band * th + y) * (uint32_t)gw + ct * tw + x);
  }
};

inline OrderGeo make_order_geo(const fva_problem& p) {
  OrderGeo g;
  g.kind = p.order_kind;
  g.n = p.seq_len;
  g.hw = p.grid_h * p.grid_w;
  g.gw = p.grid_w;
  g.gh = p.grid_h;
  g.th = p.tile_h;
  g.tw = p.tile_w;
  g.div_hw = FastDiv((uint32_t)g.hw);
  if (p.tile_h > 0) {
    g.last_h = p.grid_h - ((p.grid_h - 1) / p.tile_h) * p.tile_h;
    g.last_w = p.grid_w - ((p.grid_w - 1) / p.tile_w) * p.tile_w;
    g.div_band = FastDiv((uint32_t)(p.tile_h * p.grid_w));
    g.div_tile_full = FastDiv((uint32_t)(p.tile_h * p.tile_w));
    g.div_tile_last = FastDiv((uint32_t)(g.last_h * p.tile_w));
    g.div_w_full = FastDiv((uint32_t)p.tile_w);
    g.div_w_last = FastDiv((uint32_t)g.last_w);
  } else {
    g.last_h = g.last_w = 0;
  }
  return g;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16x2 (lo in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Layout of the re-laid-out K and V (written by the routing pass, read by the
// attention kernel), per head h with npad = nb*B positions:
//   kp[h][p][c]        = K[token order[p]][c]        (zero rows past N)
//   vt[h][s][c][j]     = V[token order[64 s + vt_key(j)]][c]
// V is transposed per 64-position sub-block s.  Column j holds key position
// vt_key(j) of the sub-block: the order in which the S^T accumulators of the
// attention kernel hold their keys (register r of a 32-key sub-tile,
// half-wave hf: key 8(r/4) + 4hf + r%4), so that 8 consecutive columns are
// exactly the keys of one lane's P^T operand and the V^T operand is one
// 16-byte LDS load.
constexpr int VT_KEYS = 64;
__host__ __device__ constexpr int vt_key(int j) {
  return 16 * (j >> 4) + 8 * ((j & 7) >> 2) + 4 * ((j >> 3) & 1) + (j & 3);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Launch-side helpers implemented in fva_api.hip.
int record_hip_error(hipError_t e, const char* what);
int device_cu_count();

}  // namespace fva
