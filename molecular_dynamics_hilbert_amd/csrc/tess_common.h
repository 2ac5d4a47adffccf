// tess_common.h -- internal definitions shared by the HIP translation units of libtess.
//
// Coupling coefficients are computed at compile time by exact integration of monomials over
// the unit sphere, so device code sees them as immediates after loop unrolling.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tess.h"

namespace tess {

// ------------------------------------------------------------------------------------
// Real spherical harmonics up to l = 2 (component normalisation, sum_m Y_lm^2 = 2l+1) as
// polynomials in the unit vector n = (x, y, z); component offset l^2 + m:
//   Y0 = 1; Y1 = sqrt3 (x, y, z);
//   Y2 = (sqrt15 xy, sqrt15 yz, sqrt5/2 (2z^2 - x^2 - y^2), sqrt15 xz, sqrt15/2 (x^2 - y^2)).
// (On the sphere 2z^2 - x^2 - y^2 = 3z^2 - 1.)
// ------------------------------------------------------------------------------------
struct Mono {
  double c;
  int a, b, d;  // c * x^a y^b z^d
};
struct Poly {
  int n;
  Mono t[3];
};

constexpr double csqrt(double x) {
  double r = x > 1.0 ? x : 1.0;
  for (int i = 0; i < 200; i++) r = 0.5 * (r + x / r);
  return r;
}

constexpr Poly sh_poly(int comp) {
  const double s3 = csqrt(3.0), s5 = csqrt(5.0), s15 = csqrt(15.0);
  switch (comp) {
    case 0: return Poly{1, {{1.0, 0, 0, 0}, {}, {}}};
    case 1: return Poly{1, {{s3, 1, 0, 0}, {}, {}}};
    case 2: return Poly{1, {{s3, 0, 1, 0}, {}, {}}};
    case 3: return Poly{1, {{s3, 0, 0, 1}, {}, {}}};
    case 4: return Poly{1, {{s15, 1, 1, 0}, {}, {}}};
    case 5: return Poly{1, {{s15, 0, 1, 1}, {}, {}}};
    case 6: return Poly{3, {{s5, 0, 0, 2}, {-0.5 * s5, 2, 0, 0}, {-0.5 * s5, 0, 2, 0}}};
    case 7: return Poly{1, {{s15, 1, 0, 1}, {}, {}}};
    default: return Poly{2, {{0.5 * s15, 2, 0, 0}, {-0.5 * s15, 0, 2, 0}, {}}};
  }
}

// (1/4pi) * integral over the unit sphere of x^a y^b z^c = (a-1)!!(b-1)!!(c-1)!!/(a+b+c+1)!!
// for even a, b, c and 0 otherwise.
constexpr double dfact(int n) { return n <= 0 ? 1.0 : n * dfact(n - 2); }
constexpr double sphere_mean(int a, int b, int c) {
  if ((a & 1) || (b & 1) || (c & 1)) return 0.0;
  return dfact(a - 1) * dfact(b - 1) * dfact(c - 1) / dfact(a + b + c + 1);
}

// Coupling paths (l1 sender degree, l2 harmonic degree, l3 output degree): all l <= LMAX
// with the triangle rule and l1+l2+l3 even, lexicographic. Tensor C^p[m1][m2][m3] = real
// Gaunt integral rescaled to Frobenius norm sqrt(2 l3 + 1).
struct CGTable {
  int P;
  int l1[11], l2[11], l3[11];
  double v[11][5][5][5];
};

constexpr CGTable make_cg(int lmax) {
  CGTable t{};
  t.P = 0;
  for (int a = 0; a <= lmax; a++)
    for (int b = 0; b <= lmax; b++)
      for (int c = 0; c <= lmax; c++) {
        int lo = a > b ? a - b : b - a;
        if (c < lo || c > a + b || ((a + b + c) & 1)) continue;
        int p = t.P++;
        t.l1[p] = a; t.l2[p] = b; t.l3[p] = c;
        double f = 0.0;
        for (int m1 = 0; m1 < 2 * a + 1; m1++)
          for (int m2 = 0; m2 < 2 * b + 1; m2++)
            for (int m3 = 0; m3 < 2 * c + 1; m3++) {
              Poly p1 = sh_poly(a * a + m1), p2 = sh_poly(b * b + m2), p3 = sh_poly(c * c + m3);
              double g = 0.0;
              for (int i = 0; i < p1.n; i++)
                for (int j = 0; j < p2.n; j++)
                  for (int k = 0; k < p3.n; k++)
                    g += p1.t[i].c * p2.t[j].c * p3.t[k].c *
                         sphere_mean(p1.t[i].a + p2.t[j].a + p3.t[k].a,
                                     p1.t[i].b + p2.t[j].b + p3.t[k].b,
                                     p1.t[i].d + p2.t[j].d + p3.t[k].d);
              t.v[p][m1][m2][m3] = g;
              f += g * g;
            }
        double s = csqrt(2.0 * c + 1.0) / csqrt(f);
        for (int m1 = 0; m1 < 5; m1++)
          for (int m2 = 0; m2 < 5; m2++)
            for (int m3 = 0; m3 < 5; m3++) {
              double v = t.v[p][m1][m2][m3] * s;
              // exact zeros stay zero; tiny round-off residues are cleared
              t.v[p][m1][m2][m3] = (v > 1e-12 || v < -1e-12) ? v : 0.0;
            }
      }
  return t;
}

constexpr CGTable kCG1 = make_cg(1);
constexpr CGTable kCG2 = make_cg(2);

template <int LMAX>
struct Dims {
  static constexpr int D = (LMAX + 1) * (LMAX + 1);
  static constexpr int P = LMAX == 1 ? 4 : 11;
};

template <int LMAX>
__device__ __forceinline__ constexpr const CGTable& cg_table() {
  if constexpr (LMAX == 1) return kCG1; else return kCG2;
}

// Bit p set for the paths with sender degree l1 == l (paths_from), or with output degree
// l3 == l (paths_to); all_paths has every bit.
template <int LMAX>
constexpr uint32_t paths_from(int l) {
  const CGTable& T = LMAX == 1 ? kCG1 : kCG2;
  uint32_t m = 0;
  for (int p = 0; p < T.P; p++)
    if (T.l1[p] == l) m |= 1u << p;
  return m;
}
template <int LMAX>
constexpr uint32_t paths_to(int l) {
  const CGTable& T = LMAX == 1 ? kCG1 : kCG2;
  uint32_t m = 0;
  for (int p = 0; p < T.P; p++)
    if (T.l3[p] == l) m |= 1u << p;
  return m;
}
template <int LMAX>
constexpr uint32_t all_paths() {
  return (1u << Dims<LMAX>::P) - 1u;
}

// Real spherical harmonics values on a unit vector (float).
template <int LMAX>
__device__ __forceinline__ void sph(float x, float y, float z, float* Y) {
  constexpr float s3 = 1.7320508075688772f, s15 = 3.8729833462074170f, s5 = 2.2360679774997896f;
  Y[0] = 1.0f;
  Y[1] = s3 * x; Y[2] = s3 * y; Y[3] = s3 * z;
  if constexpr (LMAX >= 2) {
    Y[4] = s15 * x * y;
    Y[5] = s15 * y * z;
    Y[6] = 0.5f * s5 * (3.0f * z * z - 1.0f);
    Y[7] = s15 * x * z;
    Y[8] = 0.5f * s15 * (x * x - y * y);
  }
}

// g = J_Y(n)^T Ybar (gradient of sum_d Ybar_d Y_d(n) with respect to n, polynomial form).
template <int LMAX>
__device__ __forceinline__ void sph_vjp(float x, float y, float z, const float* Yb, float* g) {
  constexpr float s3 = 1.7320508075688772f, s15 = 3.8729833462074170f, s5 = 2.2360679774997896f;
  g[0] = s3 * Yb[1];
  g[1] = s3 * Yb[2];
  g[2] = s3 * Yb[3];
  if constexpr (LMAX >= 2) {
    g[0] += s15 * (y * Yb[4] + z * Yb[7] + x * Yb[8]);
    g[1] += s15 * (x * Yb[4] + z * Yb[5] - y * Yb[8]);
    g[2] += s15 * (y * Yb[5] + x * Yb[7]) + 3.0f * s5 * z * Yb[6];
  }
}

// A[d3][d1] = sum_p w_p sum_m2 C^p[m1][m2][m3] Y[l2^2+m2]   (d3 = l3^2+m3, d1 = l1^2+m1)
template <int LMAX>
__device__ __forceinline__ void coupling_matrix(const float* w, const float* Y, float* A) {
  constexpr int D = Dims<LMAX>::D;
  constexpr const CGTable& T = cg_table<LMAX>();
#pragma unroll
  for (int k = 0; k < D * D; k++) A[k] = 0.0f;
#pragma unroll
  for (int p = 0; p < Dims<LMAX>::P; p++) {
#pragma unroll
    for (int m1 = 0; m1 < 5; m1++)
#pragma unroll
      for (int m3 = 0; m3 < 5; m3++) {
        if (m1 >= 2 * T.l1[p] + 1 || m3 >= 2 * T.l3[p] + 1) continue;
        float k = 0.0f;
        bool any = false;
#pragma unroll
        for (int m2 = 0; m2 < 5; m2++) {
          if (m2 < 2 * T.l2[p] + 1 && T.v[p][m1][m2][m3] != 0.0) {
            k += (float)T.v[p][m1][m2][m3] * Y[T.l2[p] * T.l2[p] + m2];
            any = true;
          }
        }
        if (any) A[(T.l3[p] * T.l3[p] + m3) * D + T.l1[p] * T.l1[p] + m1] += w[p] * k;
      }
  }
}

// Adjoint of coupling_matrix given Abar = dE/dA: wbar_p = <Abar, K^p>, Ybar = dE/dY.
template <int LMAX>
__device__ __forceinline__ void coupling_matrix_vjp(const float* w, const float* Y,
                                                    const float* Ab, float* wb, float* Yb) {
  constexpr int D = Dims<LMAX>::D;
  constexpr const CGTable& T = cg_table<LMAX>();
#pragma unroll
  for (int d = 0; d < D; d++) Yb[d] = 0.0f;
#pragma unroll
  for (int p = 0; p < Dims<LMAX>::P; p++) {
    float acc = 0.0f;
#pragma unroll
    for (int m2 = 0; m2 < 5; m2++) {
      if (m2 >= 2 * T.l2[p] + 1) continue;
      float tpm = 0.0f;  // sum_{m1,m3} C^p[m1][m2][m3] Abar[(l3,m3)][(l1,m1)]
      bool any = false;
#pragma unroll
      for (int m1 = 0; m1 < 5; m1++)
#pragma unroll
        for (int m3 = 0; m3 < 5; m3++) {
          if (m1 < 2 * T.l1[p] + 1 && m3 < 2 * T.l3[p] + 1 && T.v[p][m1][m2][m3] != 0.0) {
            tpm += (float)T.v[p][m1][m2][m3] *
                   Ab[(T.l3[p] * T.l3[p] + m3) * D + T.l1[p] * T.l1[p] + m1];
            any = true;
          }
        }
      if (any) {
        acc += tpm * Y[T.l2[p] * T.l2[p] + m2];
        Yb[T.l2[p] * T.l2[p] + m2] += w[p] * tpm;
      }
    }
    wb[p] = acc;
  }
}

// ---- small device helpers ----------------------------------------------------------
// Workgroups are dealt round-robin over the 8 XCDs (each with its own L2). Renumber them so
// that XCD x works through one contiguous range of logical blocks: with Hilbert-ordered
// atoms, neighbouring rows then share their gathered feature rows in that XCD's L2.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t nb) {
  const uint32_t per = nb >> 3, rem = nb & 7u, x = b & 7u, idx = b >> 3;
  return x < rem ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// Logistic function with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Exclusive scan of int32 counts in place, any length (one launch up to 16,384 entries, else
// two, or three beyond 2^24); `partial` holds ceil(n/4096) entries. With `stats` (zeroed by the
// caller when n > 16,384) the launches also write the largest count to stats[0] and the
// 64-bit total of the counts to stats[2..3] (8-byte aligned), and with `extra` a copy of
// *extra to stats[1] (read after the work before the scan on the stream). Host wrapper in
// nbr.hip.
hipError_t scan_exclusive_i32(int32_t* data, int64_t n, int32_t* partial, hipStream_t s,
                              int32_t* stats = nullptr, const int32_t* extra = nullptr);

}  // namespace tess

namespace tess {
// Host-side carving of the caller's workspace into aligned sub-arrays. With base == NULL it
// only measures.
struct Carver {
  char* base;
  int64_t off;
  template <class T>
  T* take(int64_t count) {
    off = (off + 255) & ~int64_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * (int64_t)sizeof(T);
    return p;
  }
};

// Device status word: the first word of every workspace. Kernels OR in bits for problems
// they detect on the device; the next synchronising call on the workspace reports and clears
// them (tess_check_status, tess_build_neighbors, tess_md_steps).
constexpr int32_t kStatusSpecies = 1;    // a species index outside [0, n_species)
constexpr int32_t kStatusNonFinite = 2;  // a non-finite position, energy or force
constexpr int32_t kStatusRadial = 4;     // radial MLP too rough for the interpolation table
// Error code of a status word (species first, then non-finite values), TESS_OK for 0.
inline int32_t status_error(int32_t bits) {
  return (bits & kStatusSpecies) ? TESS_ERR_SPECIES
         : (bits & kStatusNonFinite) ? TESS_ERR_NONFINITE
         : (bits & kStatusRadial) ? TESS_ERR_RADIAL
                                  : TESS_OK;
}

// Neighbour-build scratch (a prefix of every workspace).
struct NbrWS {
  float* pos_w;       // [3n] wrapped positions (pre-sort order)
  uint32_t* key[2];   // [n] ping-pong keys
  int32_t* idx[2];    // [n] ping-pong indices
  int32_t* hist;      // [256 * nblk + 1]
  int32_t* sp_tmp;    // [n]
  int32_t* pa_tmp;    // [n]
  float* v_tmp;       // [3n]
  float* f_tmp;       // [3n]
  int32_t* cell_start;  // [ncell_cap + 1]
  int32_t* cell_fill;   // [ncell_cap]
  int32_t* cell_atoms;  // [n] atom indices grouped by cell
  float4* cell_pos;     // [n] their positions (and index bits), grouped by cell
  int32_t* cell_id;     // [n]
  int32_t* scan_tmp;    // [scan partial sums]
  int32_t* misc;        // [16]: [0] max row length, [2..3] 64-bit pair count
  int64_t ncell_cap;
};
NbrWS carve_nbr(Carver& c, int32_t n);

// Internal rebuild used by tess_build_neighbors and tess_md_steps. Optional extra arrays
// are permuted along (forces [n][3], perm_accum [n]).
// `status` is the workspace's device status word (see below): the wrap kernel sets
// kStatusNonFinite for a non-finite coordinate, and the call reads the word at its one
// synchronisation and returns TESS_ERR_SPECIES / TESS_ERR_NONFINITE (clearing it) when a bit
// is set, before the fill pass.
int32_t build_neighbors_impl(int32_t n, const float box[3], float r_cut, float skin,
                             float* pos, int32_t* species, float* vel, float* ref_pos,
                             float* forces, int32_t* perm_accum, int32_t* perm, uint32_t* hkey,
                             int32_t* row_ptr, uint32_t* col_shift, int32_t* rev,
                             int64_t edge_cap, int64_t* n_edges, const NbrWS& ws,
                             int32_t* status, hipStream_t stream);
// Reverse-pair index of a sorted CSR (rev[e] = slot of (j <- i, -s)).
hipError_t rev_index(int32_t n, const int32_t* row_ptr, const uint32_t* col, int32_t* rev,
                     hipStream_t s);

// Energy/force pass (model.hip). ws points at the energy/force part of the workspace, laid
// out for `ecap` edges.
bool ef_shape_supported(const tess_model_desc& md);
int64_t ef_workspace_bytes(const tess_model_desc& md, int32_t n, int64_t ecap);
int32_t ef_dispatch(const tess_model_desc& md, const float* weights, int32_t n, const float box[3],
                    const float* pos, const int32_t* species, const int32_t* row_ptr,
                    const uint32_t* col_shift, const int32_t* rev, int64_t n_edges,
                    int64_t ecap, double* energy, float* e_atom, float* forces, char* ws,
                    int64_t ws_bytes, int32_t* status, hipStream_t st,
                    uint32_t* rmin2_bits = nullptr);
}  // namespace tess

#define TESS_HIP_CHECK(expr)                       \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return TESS_ERR_HIP;     \
  } while (0)

// Optional per-kernel timing (tess_timing_enable / tess_timing_read): HIP events recorded on
// the launching stream around each instrumented launch.
namespace tess {
// Space-filling curve of the atom order: 0 Hilbert (the method's), 1 Morton (comparisons).
int sort_curve();
bool timing_on();
bool timing_wants(const char* name);
void timing_mark(const char* name, hipStream_t st, bool begin);
}  // namespace tess
#define TESS_TIMED(name, st, ...)            \
  do {                                       \
    if (tess::timing_wants(name)) {          \
      tess::timing_mark(name, st, true);     \
      __VA_ARGS__;                           \
      tess::timing_mark(name, st, false);    \
    } else {                                 \
      __VA_ARGS__;                           \
    }                                        \
  } while (0)
