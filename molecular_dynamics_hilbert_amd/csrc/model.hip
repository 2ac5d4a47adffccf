// model.hip -- energy and forces of the equivariant message-passing attention stack on
// gfx950 (Tessera title and abstract: equivariant attention layers, forces by
// back-propagation; the backward pass is the per-layer vector-Jacobian-product chain that the
// REANN-MPI review describes, key_machinery field).
//
// Data layout in HBM (fp32): node features [N][D][C] (component-major per node, channels
// contiguous, so a wave reading one component of one node reads 4C contiguous bytes);
// q|k per node [N][2C]; per active edge (r < r_cut, destination-major) geometry float4
// (r_vec, |r|) and, per layer, path-major rows of radial weights w_p and dw_p/dr, and logits
// s[4].
//
// Once per pass: the radial MLP of every layer tabulated over r (fp64 knots) and interpolated
// for every active edge (cubic Hermite, C^1). Kernels per layer (forward): MFMA GEMM q|k and
// the logits kernel; edge contraction (one wave per destination row: softmax statistics,
// coupling matrices A_e into LDS, then alpha * A_e h_j summed over the row's edges on 4x4x1
// MFMA blocks); MFMA GEMMs of the gated residual update with fused epilogues. Backward:
// elementwise update adjoint + MFMA GEMMs; edge_grad (one lane per edge and head: per-head
// sum over channels of mbar_i (x) h_j contracted through the coupling adjoint, giving the
// logit adjoint and dE/dr_vec); the transposed edge contraction (one wave per row: h_bar via
// A^T); the q/k adjoints (k_qk_bar) and their MFMA GEMM; force assembly through the
// reverse-edge index.
#include "tess_common.h"

#include <vector>

namespace tess {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr float kPi = 3.14159265358979323846f;
constexpr int kRadKnots = 1024;  // intervals of the radial-weight table over [0, r_c]

inline int32_t gridn(int64_t n, int b) { return (int32_t)((n + b - 1) / b); }

// ---------------------------------------------------------------------------------------
// GEMM: Y[r][o] = sum_k X[r][k] * Wt[k][o] (fp32 MFMA 32x32x2), with row maps so that the
// same kernel reads one irrep block of [N][D][C] features.
// ---------------------------------------------------------------------------------------
struct RowMap {
  int64_t nstride;  // floats between nodes
  int32_t cstride;  // floats between components of one node
  int32_t c0;       // first component
  int32_t rpn;      // rows per node (components of the block)
};
__device__ __forceinline__ int64_t row_off(const RowMap& m, int64_t r) {
  int64_t n = r / m.rpn;
  int32_t k = (int32_t)(r - n * m.rpn);
  return n * m.nstride + (int64_t)(m.c0 + k) * m.cstride;
}

enum { EPI_STORE = 0, EPI_ADD = 1, EPI_UPD0 = 2, EPI_UPDL = 3 };

struct Epi {
  float* y;           // output (store/add), or pre-activation store for UPD*
  RowMap ym;
  const float* hin;   // UPD*: residual input features (UPDL: NULL means zero)
  float* hout;        // UPD*: output features
  RowMap hm;          // UPD*: map of hin/hout rows
  const float* gates; // UPDL: [N][C(1+Lm)] pre-activations (gate of degree l at l*C)
  int32_t gstride, goff, cdim;
};

// Block tile 128 rows x 64 columns, 4 waves of 32 x 64 (two 32x32 MFMA tiles each). The
// block's K x 64 slice of Wt is staged in LDS once, while the block's X rows are in flight.
// The MFMAs form the transposed tile (Wt^T X^T), so that a lane ends with 16 columns of ONE
// output row, in four runs of 4 consecutive columns: the epilogue then reads its inputs and
// writes its outputs as float4 at one row offset per lane (a layout with a column per lane
// would need 4x as many scalar memory instructions and a row offset per element). Each lane
// loads its row of X with float4 loads: lanes 0-31 take k = 8s..8s+3 and lanes 32-63
// k = 8s+4..8s+7, so MFMA step (s, q) pairs k = 8s+q (first half-wave) with k = 8s+4+q
// (second half-wave), and the Wt operand uses the same pairing. K must be a multiple of 16
// and at most kGemmMaxK; O, the row maps' strides and offsets, the gate stride and offset and
// cdim are multiples of 4 and the arrays 16-byte aligned (checked by the launcher, except the
// alignment of the base pointers, which are workspace or weight-blob carvings).
constexpr int kGemmMaxK = 192;

template <int EPI, int K>
__global__ void __launch_bounds__(256) k_gemm(int64_t M, int O, const float* __restrict__ X,
                                              RowMap xm, const float* __restrict__ Wt, Epi ep) {
  static_assert(K % 16 == 0 && K <= kGemmMaxK, "K is a multiple of 16, at most kGemmMaxK");
  __shared__ float Ws[K][64 + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 128 + w * 32 + col;
  const int o0 = blockIdx.y * 64;
  const bool row_ok = row < M;
  const int kh = hf * 4;
  float4 xa[K / 8];
  if (row_ok) {
    const float* xr = X + row_off(xm, row);
#pragma unroll
    for (int s8 = 0; s8 < K / 8; s8++) xa[s8] = *reinterpret_cast<const float4*>(xr + 8 * s8 + kh);
  } else {
#pragma unroll
    for (int s8 = 0; s8 < K / 8; s8++) xa[s8] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // the block's K x 64 slice of Wt, staged after the X rows are requested (rows of Wt are O
  // floats, O a multiple of 4, and the blob is 16-byte aligned)
  // (every load is requested before the first LDS write)
  {
    float4 wv[K / 16];
#pragma unroll
    for (int i = 0; i < K / 16; i++) {
      const int k = t + 256 * i, kk = k >> 4, oo = 4 * (k & 15);
      wv[i] = *reinterpret_cast<const float4*>(Wt + (int64_t)kk * O + (o0 + oo < O ? o0 + oo : 0));
    }
#pragma unroll
    for (int i = 0; i < K / 16; i++) {
      const int k = t + 256 * i, kk = k >> 4, oo = 4 * (k & 15);
      const float4 v = o0 + oo < O ? wv[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      Ws[kk][oo] = v.x;
      Ws[kk][oo + 1] = v.y;
      Ws[kk][oo + 2] = v.z;
      Ws[kk][oo + 3] = v.w;
    }
  }
  // this lane's output row (clamped past M so that the loads below stay in bounds): its
  // offsets in y, h and the gates, with one 32-bit division by the rows-per-node count (the
  // row maps of y and h share it)
  const uint32_t rr = (uint32_t)(row_ok ? row : M - 1);
  const uint32_t rpn = (uint32_t)ep.ym.rpn;
  const uint32_t nd = rr / rpn;
  const int32_t kc = (int32_t)(rr - nd * rpn);
  const int64_t yb = (int64_t)nd * ep.ym.nstride + (int64_t)(ep.ym.c0 + kc) * ep.ym.cstride;
  const int64_t hb = (int64_t)nd * ep.hm.nstride + (int64_t)(ep.hm.c0 + kc) * ep.hm.cstride;
  const int64_t gb = (int64_t)nd * ep.gstride + ep.goff;
  // epilogue inputs at columns o0 + 32 nt + 8 g + 4 hf .. + 3, requested before the MFMA
  // loop from clamped columns (a load under a branch would be waited for inside the branch);
  // values of columns outside the output are never used
  float4 in0[2][4], in1[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; nt++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int oc = o0 + 32 * nt + 8 * g + 4 * hf;
      const bool ok = oc < O;
      const bool hok = ok && (EPI != EPI_UPD0 || oc < ep.cdim);
      in0[nt][g] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      in1[nt][g] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (EPI == EPI_ADD) in0[nt][g] = *reinterpret_cast<const float4*>(ep.y + yb + (ok ? oc : 0));
      if (EPI == EPI_UPD0 || EPI == EPI_UPDL)  // a NULL residual input reads as zero
        if (ep.hin) in0[nt][g] = *reinterpret_cast<const float4*>(ep.hin + hb + (hok ? oc : 0));
      if (EPI == EPI_UPDL)
        in1[nt][g] = *reinterpret_cast<const float4*>(ep.gates + gb + (ok ? oc : 0));
    }
  __syncthreads();
  floatx16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; v++) { acc0[v] = 0.0f; acc1[v] = 0.0f; }
#pragma unroll
  for (int s8 = 0; s8 < K / 8; s8++) {
    const float av[4] = {xa[s8].x, xa[s8].y, xa[s8].z, xa[s8].w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int k = 8 * s8 + q + kh;
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(Ws[k][col], av[q], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(Ws[k][32 + col], av[q], acc1, 0, 0, 0);
    }
  }
  // Epilogue: register v = 4 g + s of tile nt holds column o0 + 32 nt + 8 g + 4 hf + s of this
  // lane's row.
  if (!row_ok) return;
#pragma unroll
  for (int nt = 0; nt < 2; nt++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int oc = o0 + 32 * nt + 8 * g + 4 * hf;
      if (oc >= O) continue;
      const floatx16& a = nt == 0 ? acc0 : acc1;
      const float4 v = make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
      float4* yp = reinterpret_cast<float4*>(ep.y + yb + oc);
      const float4 x0 = in0[nt][g];
      if (EPI == EPI_STORE) {
        *yp = v;
      } else if (EPI == EPI_ADD) {
        *yp = make_float4(x0.x + v.x, x0.y + v.y, x0.z + v.z, x0.w + v.w);
      } else if (EPI == EPI_UPD0) {
        *yp = v;
        if (oc < ep.cdim)
          *reinterpret_cast<float4*>(ep.hout + hb + oc) =
              make_float4(x0.x + v.x * sigmoidf_(v.x), x0.y + v.y * sigmoidf_(v.y),
                          x0.z + v.z * sigmoidf_(v.z), x0.w + v.w * sigmoidf_(v.w));
      } else {  // EPI_UPDL
        const float4 x1 = in1[nt][g];
        *yp = v;
        *reinterpret_cast<float4*>(ep.hout + hb + oc) =
            make_float4(x0.x + sigmoidf_(x1.x) * v.x, x0.y + sigmoidf_(x1.y) * v.y,
                        x0.z + sigmoidf_(x1.z) * v.z, x0.w + sigmoidf_(x1.w) * v.w);
      }
    }
}

// o_first: when > 0, only output columns [0, o_first) are computed (O stays the row length of
// Wt and of the outputs).
template <int EPI>
hipError_t gemm(hipStream_t st, int64_t M, int K, int O, const float* X, RowMap xm,
                const float* Wt, const Epi& ep, int o_first = 0) {
  if (M <= 0) return hipSuccess;
  // the kernel moves rows of Wt, y, h and the gates in float4 pieces
  auto q4 = [](int64_t v) { return (v & 3) == 0; };
  auto map4 = [&](const RowMap& m) { return q4(m.nstride) && q4((int64_t)m.c0 * m.cstride) && q4(m.cstride); };
  if (!q4(O) || !map4(ep.ym) || (EPI >= EPI_UPD0 && (!map4(ep.hm) || !q4(ep.cdim))) ||
      (EPI == EPI_UPDL && (!q4(ep.gstride) || !q4(ep.goff))))
    return hipErrorInvalidValue;
  dim3 g((unsigned)((M + 127) / 128), (unsigned)(((o_first > 0 ? o_first : O) + 63) / 64));
  switch (K) {
    case 16: TESS_TIMED("node_gemm", st, k_gemm<EPI, 16><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 32: TESS_TIMED("node_gemm", st, k_gemm<EPI, 32><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 48: TESS_TIMED("node_gemm", st, k_gemm<EPI, 48><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 64: TESS_TIMED("node_gemm", st, k_gemm<EPI, 64><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 96: TESS_TIMED("node_gemm", st, k_gemm<EPI, 96><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 128: TESS_TIMED("node_gemm", st, k_gemm<EPI, 128><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    case 192: TESS_TIMED("node_gemm", st, k_gemm<EPI, 192><<<g, 256, 0, st>>>(M, O, X, xm, Wt, ep)); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Weight preparation: transposed copies for the forward GEMMs, every layer in one launch
// (blockIdx.y = layer). Per layer of the blob (row-major [out][in]): W_q, W_k, W1, W2, W_lin0,
// W_lin^l; written as [W_q^T | W_k^T] ([C][2C]), W_lin0^T ([C][G]) and W_lin^l^T ([C][C]).
// ---------------------------------------------------------------------------------------
// Small fills (used instead of memset nodes so the pass can be captured in a HIP graph).
__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) p[k] = v;
}
__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) p[k] = v;
}

template <int LMAX, int C, int R>
__global__ void k_prep_weights(const float* __restrict__ weights, int S, int K,
                               float* __restrict__ WqkT, float* __restrict__ W0T,
                               float* __restrict__ WlT) {
  constexpr int P = Dims<LMAX>::P;
  constexpr int G = C * (1 + LMAX);
  constexpr int NEL = 2 * C * C + G * C + LMAX * C * C;
  const int t = blockIdx.y;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= NEL) return;
  const int64_t stride = 2 * C * C + (int64_t)R * K + P * R + G * C + LMAX * C * C;
  const float* lb = weights + (int64_t)S * C + t * stride;
  const float* lin = lb + 2 * C * C + (int64_t)R * K + P * R;  // W_lin0, then W_lin^l
  if (k < 2 * C * C) {
    const int which = k / (C * C), kk = k % (C * C), r = kk / C, c = kk % C;
    WqkT[(int64_t)t * C * 2 * C + c * 2 * C + which * C + r] = lb[k];
  } else if (k < 2 * C * C + G * C) {
    const int kk = k - 2 * C * C, r = kk / C, c = kk % C;
    W0T[(int64_t)t * C * G + c * G + r] = lin[kk];
  } else {
    const int kk = k - 2 * C * C - G * C, l1 = kk / (C * C), k2 = kk % (C * C), r = k2 / C,
              c = k2 % C;
    WlT[((int64_t)t * LMAX + l1) * C * C + c * C + r] = lin[G * C + kk];
  }
}

// h^0: the species embedding in the l = 0 component. The l >= 1 components of h^0 are zero
// and never read (layer 0 contracts only l = 0 inputs and its gated update starts from zero).
// Species index clamped to [0, S): an index out of range gives wrong values, never an access
// outside the weights.
__device__ __forceinline__ int sp_index(int32_t s, int S) { return min(max(s, 0), S - 1); }

// An index out of range also sets kStatusSpecies in the status word (reported by the next
// synchronising call).
__global__ void k_embed(int32_t n, int C, int D, int S, const int32_t* __restrict__ species,
                        const float* __restrict__ emb, float* __restrict__ h,
                        int32_t* __restrict__ status) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (int64_t)n * C) return;
  int64_t i = k / C;
  int c = (int)(k - i * C);
  const int32_t s = species[i];
  if (c == 0 && (s < 0 || s >= S)) atomicOr(status, kStatusSpecies);
  h[i * D * C + c] = emb[sp_index(s, S) * C + c];
}

// ---------------------------------------------------------------------------------------
// Active-edge list (pairs with r < r_cut), destination-major, with geometry in fp32:
// r_vec = x_j - x_i + s L. The test is symmetric under (i,j,s) -> (j,i,-s) bit for bit.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float4 edge_vec(const float* __restrict__ pos, int32_t i, uint32_t c,
                                           float Lx, float Ly, float Lz, int32_t* j_out) {
  int32_t j = (int32_t)(c & 0x7FFFFFFu);
  int code = (int)(c >> 27);
  float sx = (float)(code / 9 - 1), sy = (float)((code / 3) % 3 - 1), sz = (float)(code % 3 - 1);
  float rx = (pos[3 * j] - pos[3 * i]) + sx * Lx;
  float ry = (pos[3 * j + 1] - pos[3 * i + 1]) + sy * Ly;
  float rz = (pos[3 * j + 2] - pos[3 * i + 2]) + sz * Lz;
  *j_out = j;
  return make_float4(rx, ry, rz, __fmul_rn(rx, rx) + __fmul_rn(ry, ry) + __fmul_rn(rz, rz));
}

__global__ void __launch_bounds__(256) k_active_count(int32_t n, const float* __restrict__ pos,
                                                      const int32_t* __restrict__ row_ptr,
                                                      const uint32_t* __restrict__ col, float Lx,
                                                      float Ly, float Lz, float rc2,
                                                      int32_t* __restrict__ acnt,
                                                      uint32_t* __restrict__ rmin2_bits) {
  int32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) acnt[n] = 0;  // entry n (the scan's total)
  if (i >= n) return;
  int cnt = 0;
  float mn = INFINITY;
  for (int32_t e = row_ptr[i] + lane; e < row_ptr[i + 1]; e += 64) {
    int32_t j;
    float4 r = edge_vec(pos, i, col[e], Lx, Ly, Lz, &j);
    const bool act = r.w < rc2;
    cnt += act;
    if (act) mn = fminf(mn, r.w);
  }
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) acnt[i] = cnt;
  if (rmin2_bits) {
    // shortest squared pair distance: non-negative floats order like their bit patterns
    for (int o = 32; o >= 1; o >>= 1) mn = fminf(mn, __shfl_xor(mn, o, 64));
    if (lane == 0 && mn < INFINITY) atomicMin(rmin2_bits, __float_as_uint(mn));
  }
}

__global__ void __launch_bounds__(256) k_active_fill(int32_t n, const float* __restrict__ pos,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const uint32_t* __restrict__ col, float Lx,
                                                     float Ly, float Lz, float rc2,
                                                     const int32_t* __restrict__ arow,
                                                     int32_t* __restrict__ adst,
                                                     int32_t* __restrict__ asrc,
                                                     int32_t* __restrict__ aslot,
                                                     int32_t* __restrict__ slot2act,
                                                     float4* __restrict__ ageo,
                                                     float* __restrict__ ar) {
  int32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (i >= n) return;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t a0 = arow[i];
  for (int32_t e0 = row_ptr[i]; e0 < row_ptr[i + 1]; e0 += 64) {
    int32_t e = e0 + lane;
    bool ok = e < row_ptr[i + 1];
    bool act = false;
    int32_t j = 0;
    float4 r = make_float4(0, 0, 0, 0);
    if (ok) {
      r = edge_vec(pos, i, col[e], Lx, Ly, Lz, &j);
      act = r.w < rc2;
    }
    uint64_t m = __ballot(act);
    if (act) {
      int32_t a = a0 + __popcll(m & lt);
      adst[a] = i;
      asrc[a] = j;
      aslot[a] = e;
      const float rr = sqrtf(r.w);
      ageo[a] = make_float4(r.x, r.y, r.z, rr);
      ar[a] = rr;
      slot2act[e] = a;
    } else if (ok) {
      slot2act[e] = -1;
    }
    a0 += __popcll(m);
  }
}

__global__ void k_active_rev(const int32_t* __restrict__ arow_n, const int32_t* __restrict__ aslot,
                             const int32_t* __restrict__ rev, const int32_t* __restrict__ slot2act,
                             int32_t* __restrict__ arev, int64_t cap) {
  int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= cap || a >= *arow_n) return;
  arev[a] = slot2act[rev[aslot[a]]];
}

// ---------------------------------------------------------------------------------------
// Radial part: cosine envelope u(r) = (cos(pi r/rc)+1)/2 and Bessel basis
// b_k = u sqrt(2/rc) sin(k pi r/rc)/r, k = 1..8, with r-derivatives.
// ---------------------------------------------------------------------------------------
struct RadialOut {
  float u, du;
  float b[8], db[8];
};
__device__ __forceinline__ void radial8(float r, float rc, RadialOut& o) {
  // 1/rc and sqrt(2/rc) are the same for every lane; 1/r uses the hardware reciprocal
  const float wk = kPi / rc;
  const float th = wk * r;
  float s1, c1;
  __sincosf(th, &s1, &c1);
  o.u = 0.5f * (c1 + 1.0f);
  o.du = -0.5f * wk * s1;
  const float pref = sqrtf(2.0f / rc);
  const float ir = __builtin_amdgcn_rcpf(r);
  float sk = s1, ck = c1;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const float a = (float)(k + 1) * wk;
    float B = pref * sk * ir;
    float dB = pref * (a * ck * ir - sk * ir * ir);
    o.b[k] = o.u * B;
    o.db[k] = o.du * B + o.u * dB;
    float sn = sk * c1 + ck * s1;
    float cn = ck * c1 - sk * s1;
    sk = sn;
    ck = cn;
  }
}

// ---------------------------------------------------------------------------------------
// Radial weights as a function of r. Every layer's radial MLP, w_p(r) = sum_h W2[p][h]
// SiLU(sum_k W1[h][k] b_k(r)) with the enveloped Bessel basis b_k, and its r-derivative are
// evaluated in fp64 at the knots r_i = i h, h = r_c / kRadKnots (one thread per knot and
// layer; at r = 0 the basis takes its limit). The edge kernel below interpolates each pair
// distance with the cubic Hermite polynomial through the two neighbouring knots' values and
// derivatives, so w is C^1 in r and dw/dr is the exact derivative of the interpolant (forces
// stay the gradient of the energy that is computed). Interpolation error for the 4-layer,
// R = 64 model with 1024 intervals: below 6e-10 of max|w| and 2e-7 of max|dw/dr| (fp64 check
// against the MLP at 2e5 random distances), about fp32 rounding.
// Table layout: [layer][knot][24]: w_0..w_11 (zero past P), then dw_0..dw_11.
// ---------------------------------------------------------------------------------------
// The radial MLP of one layer and its r-derivative in fp64 at distance r (r = 0: the basis
// takes its limit).
template <int P>
__device__ void radial_mlp_fp64(const float* __restrict__ W1, const float* __restrict__ W2,
                                int R, double rcd, double r, double* w, double* dw) {
  const double wk = 3.14159265358979323846 / rcd, pref = sqrt(2.0 / rcd);
  const double u = 0.5 * (cos(wk * r) + 1.0), du = -0.5 * wk * sin(wk * r);
  double b[8], db[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const double a = (double)(k + 1) * wk;
    double B, dB;
    if (r == 0.0) {  // sin(a r)/r -> a, and its derivative -> 0
      B = pref * a;
      dB = 0.0;
    } else {
      const double sa = sin(a * r), ca = cos(a * r);
      B = pref * sa / r;
      dB = pref * (a * ca / r - sa / (r * r));
    }
    b[k] = u * B;
    db[k] = du * B + u * dB;
  }
#pragma unroll
  for (int p = 0; p < P; p++) { w[p] = 0.0; dw[p] = 0.0; }
  for (int h = 0; h < R; h++) {
    double z = 0.0, dz = 0.0;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      z += (double)W1[h * 8 + k] * b[k];
      dz += (double)W1[h * 8 + k] * db[k];
    }
    const double sg = 1.0 / (1.0 + exp(-z));
    const double act = z * sg, dact = sg * (1.0 + z * (1.0 - sg)) * dz;
#pragma unroll
    for (int p = 0; p < P; p++) {
      w[p] += (double)W2[p * R + h] * act;
      dw[p] += (double)W2[p * R + h] * dact;
    }
  }
}

template <int P>
__global__ void __launch_bounds__(256) k_radial_table(const float* __restrict__ W1_0,
                                                      int64_t lstride, int R, float rc,
                                                      float* __restrict__ tab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // knot
  const int t = blockIdx.y;                             // layer
  if (i > kRadKnots) return;
  const float* W1 = W1_0 + (int64_t)t * lstride;  // [R][8]
  const float* W2 = W1 + (int64_t)R * 8;          // [P][R]
  const double rcd = (double)rc;
  double w[P], dw[P];
  radial_mlp_fp64<P>(W1, W2, R, rcd, (double)i * (rcd / kRadKnots), w, dw);
  float* o = tab + ((int64_t)t * (kRadKnots + 1) + i) * 24;
#pragma unroll
  for (int p = 0; p < 12; p++) {
    o[p] = p < P ? (float)w[p] : 0.0f;
    o[12 + p] = p < P ? (float)dw[p] : 0.0f;
  }
}

// Guard of the table: at the midpoint of every interval the exact MLP (fp64) is compared with
// the Hermite interpolant of the stored (fp32) knots, evaluated in fp64. Per layer the largest
// deviations of w and dw/dr and the largest |w|, |dw/dr| there are kept as float bits
// (non-negative floats order like their bit patterns) in acc[4 t .. 4 t + 3].
template <int P>
__global__ void __launch_bounds__(256) k_radial_check(const float* __restrict__ W1_0,
                                                      int64_t lstride, int R, float rc,
                                                      const float* __restrict__ tab,
                                                      uint32_t* __restrict__ acc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // interval
  const int t = blockIdx.y;                             // layer
  float ew = 0.0f, ed = 0.0f, mw = 0.0f, md = 0.0f;
  if (i < kRadKnots) {
    const float* W1 = W1_0 + (int64_t)t * lstride;
    const float* W2 = W1 + (int64_t)R * 8;
    const double rcd = (double)rc, h = rcd / kRadKnots;
    double w[P], dw[P];
    radial_mlp_fp64<P>(W1, W2, R, rcd, ((double)i + 0.5) * h, w, dw);
    const float* k0 = tab + ((int64_t)t * (kRadKnots + 1) + i) * 24;
    const float* k1 = k0 + 24;
    // cubic Hermite at t = 1/2: w = (w0 + w1)/2 + h (g0 - g1)/8; dw = 1.5 (w1 - w0)/h - (g0 + g1)/4
#pragma unroll
    for (int p = 0; p < P; p++) {
      const double w0 = k0[p], w1 = k1[p], g0 = k0[12 + p], g1 = k1[12 + p];
      const double wi = 0.5 * (w0 + w1) + 0.125 * h * (g0 - g1);
      const double di = 1.5 * (w1 - w0) / h - 0.25 * (g0 + g1);
      ew = fmaxf(ew, (float)fabs(wi - w[p]));
      ed = fmaxf(ed, (float)fabs(di - dw[p]));
      mw = fmaxf(mw, (float)fabs(w[p]));
      md = fmaxf(md, (float)fabs(dw[p]));
    }
  }
  ew = wave_max(ew); ed = wave_max(ed); mw = wave_max(mw); md = wave_max(md);
  if ((threadIdx.x & 63) == 0) {
    atomicMax(acc + 4 * t, __float_as_uint(ew));
    atomicMax(acc + 4 * t + 1, __float_as_uint(ed));
    atomicMax(acc + 4 * t + 2, __float_as_uint(mw));
    atomicMax(acc + 4 * t + 3, __float_as_uint(md));
  }
}

// Flags kStatusRadial when some layer's midpoint deviation exceeds 1e-6 of max|w| or 1e-4 of
// max|dw/dr| (for the random-init models: about 6e-10 and 2e-7), i.e. when the radial network
// is too rough for the table's knot spacing. One thread per layer.
__global__ void k_radial_verdict(int T, const uint32_t* __restrict__ acc,
                                 int32_t* __restrict__ status) {
  const int t = threadIdx.x;
  if (t >= T) return;
  const float ew = __uint_as_float(acc[4 * t]), ed = __uint_as_float(acc[4 * t + 1]);
  const float mw = __uint_as_float(acc[4 * t + 2]), md = __uint_as_float(acc[4 * t + 3]);
  if (!(ew <= 1e-6f * mw) || !(ed <= 1e-4f * md)) atomicOr(status, kStatusRadial);
}

// Radial weights w and dw/dr of layers t_begin..t_end-1 for each active edge from the table, written at
// [layer][path][edge] (path-major rows of ews floats, ews a multiple of 64); with l0tab, also
// the first layer's logits from the species table. The distances are random, so the table is
// read from LDS: persistent blocks (one per CU) take contiguous ranges of whole groups of 4
// edges, stage one layer's table (98 KB) at a time and interpolate every edge of their range
// from it. A thread takes 4 consecutive edges at a time, so each output row gets one 16-byte
// store per thread (a wave writes 1 KB of a row); slots past the active count in the last
// group get the value at r = 0 (never read). Only the paths the layer's edge kernels read are
// written: in the first layer (input features of degree 0) the paths with sender degree 0
// (mfirst), in the last layer (only the degree-0 output is used) those with output degree 0
// (mlast); the other rows of those layers are left as they are and never read.
constexpr int kRadThreads = 1024;
constexpr int kRadBlocks = 256;  // one per compute unit (the table fills most of a CU's LDS)
template <int NP>
__global__ void __launch_bounds__(kRadThreads) k_edge_radial(
    const int32_t* __restrict__ arow_n, const float* __restrict__ ar,
    const float* __restrict__ rtab, int t_begin, int t_end, float rc, float* __restrict__ ew,
    float* __restrict__ edw, int64_t lstride, int64_t ews, int64_t cap,
    const int32_t* __restrict__ adst, const int32_t* __restrict__ asrc,
    const int32_t* __restrict__ species, const float4* __restrict__ l0tab, int S,
    float4* __restrict__ es, uint32_t mfirst, uint32_t mlast) {
  __shared__ float4 stab[(kRadKnots + 1) * 6];
  const int64_t n_act = min((int64_t)*arow_n, cap);
  const int64_t ngr = (n_act + 3) / 4;  // groups of 4 edges
  const int64_t per = (ngr + gridDim.x - 1) / gridDim.x;
  const int64_t g0 = (int64_t)blockIdx.x * per, g1 = min(g0 + per, ngr);
  const float hk = rc / (float)kRadKnots, ih = (float)kRadKnots / rc;
  for (int t = t_begin; t < t_end; t++) {
    // paths whose weights the layer's kernels read (first layer: mfirst; last: mlast)
    const uint32_t pm = t == 0 ? mfirst : (t == t_end - 1 ? mlast : 0xFFFFFFFFu);
    if (t > t_begin) __syncthreads();
    const float4* src = reinterpret_cast<const float4*>(rtab + (int64_t)t * (kRadKnots + 1) * 24);
    for (int k = threadIdx.x; k < (kRadKnots + 1) * 6; k += kRadThreads) stab[k] = src[k];
    __syncthreads();
    // |r| of the thread's next group of 4 edges is requested before the current one is used
    int64_t g = g0 + threadIdx.x;
    float4 rn = g < g1 ? *reinterpret_cast<const float4*>(ar + 4 * g) : make_float4(0, 0, 0, 0);
    for (; g < g1; g += kRadThreads) {
      const int64_t a = 4 * g;
      const float4 r4 = rn;
      if (g + kRadThreads < g1) rn = *reinterpret_cast<const float4*>(ar + 4 * (g + kRadThreads));
      const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
      // cubic Hermite basis on [r_i, r_i + h] of each of the 4 edges, and its r-derivative
      float hb[4][8];
      int ib[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float r = a + e < n_act ? rv[e] : 0.0f;
        const float x = r * ih;
        const int i = min(max((int)x, 0), kRadKnots - 1);
        const float tt = x - (float)i, t2 = tt * tt, t3 = t2 * tt;
        ib[e] = i;
        hb[e][0] = 2.0f * t3 - 3.0f * t2 + 1.0f;
        hb[e][1] = (t3 - 2.0f * t2 + tt) * hk;
        hb[e][2] = 3.0f * t2 - 2.0f * t3;
        hb[e][3] = (t3 - t2) * hk;
        hb[e][4] = 6.0f * (t2 - tt) * ih;
        hb[e][5] = 3.0f * t2 - 4.0f * tt + 1.0f;
        hb[e][6] = -hb[e][4];
        hb[e][7] = 3.0f * t2 - 2.0f * tt;
      }
      // paths in groups of 4: one 16-byte store per output row per thread
      float* pw = ew + t * lstride + a;
      float* pd = edw + t * lstride + a;
#pragma unroll
      for (int q = 0; q < (NP + 3) / 4; q++) {
        if (((pm >> (4 * q)) & 15u) == 0u) {  // block-uniform: no path of the group is read
          pw += 4 * ews;
          pd += 4 * ews;
          continue;
        }
        float wv[4][4], dv[4][4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float4* k0 = stab + ib[e] * 6;
          const float4 w0 = k0[q], g0v = k0[3 + q], w1 = k0[6 + q], g1v = k0[9 + q];
          const float* h = hb[e];
          wv[e][0] = h[0] * w0.x + h[1] * g0v.x + h[2] * w1.x + h[3] * g1v.x;
          wv[e][1] = h[0] * w0.y + h[1] * g0v.y + h[2] * w1.y + h[3] * g1v.y;
          wv[e][2] = h[0] * w0.z + h[1] * g0v.z + h[2] * w1.z + h[3] * g1v.z;
          wv[e][3] = h[0] * w0.w + h[1] * g0v.w + h[2] * w1.w + h[3] * g1v.w;
          dv[e][0] = h[4] * w0.x + h[5] * g0v.x + h[6] * w1.x + h[7] * g1v.x;
          dv[e][1] = h[4] * w0.y + h[5] * g0v.y + h[6] * w1.y + h[7] * g1v.y;
          dv[e][2] = h[4] * w0.z + h[5] * g0v.z + h[6] * w1.z + h[7] * g1v.z;
          dv[e][3] = h[4] * w0.w + h[5] * g0v.w + h[6] * w1.w + h[7] * g1v.w;
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
          if (4 * q + c < NP) {
            if ((pm >> (4 * q + c)) & 1u) {
              *reinterpret_cast<float4*>(pw) = make_float4(wv[0][c], wv[1][c], wv[2][c], wv[3][c]);
              *reinterpret_cast<float4*>(pd) = make_float4(dv[0][c], dv[1][c], dv[2][c], dv[3][c]);
            }
            pw += ews;
            pd += ews;
          }
        }
      }
      if (t == 0 && l0tab) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if (a + e < n_act) {
            const int si = sp_index(species[adst[a + e]], S);
            const int sj = sp_index(species[asrc[a + e]], S);
            es[a + e] = l0tab[si * S + sj];
          }
        }
      }
    }
  }
}

// First layer: the input features are the species embedding, so q = W_q e_s and k = W_k e_s
// take one value per species and the logits one value per (destination species, source
// species) pair: tab[s_i S + s_j].h = <q_(s_i)^h, k_(s_j)^h>/sqrt(d) (heads past H are 0).
// One block.
template <int C, int H>
__global__ void __launch_bounds__(256) k_l0_logits(int S, const float* __restrict__ emb,
                                                   const float* __restrict__ Wq,
                                                   const float* __restrict__ Wk,
                                                   float4* __restrict__ tab) {
  constexpr int dh = C / H;
  __shared__ float sq[16][C], sk[16][C];
  for (int t = threadIdx.x; t < S * C; t += blockDim.x) {
    const int sp = t / C, c = t % C;
    float q = 0.0f, k = 0.0f;
    for (int c2 = 0; c2 < C; c2++) {
      q += Wq[c * C + c2] * emb[sp * C + c2];
      k += Wk[c * C + c2] * emb[sp * C + c2];
    }
    sq[sp][c] = q;
    sk[sp][c] = k;
  }
  __syncthreads();
  const float isd = rsqrtf((float)dh);
  for (int t = threadIdx.x; t < S * S; t += blockDim.x) {
    const int si = t / S, sj = t % S;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < C; c++) v[c / dh] += sq[si][c] * sk[sj][c];
    tab[t] = make_float4(v[0] * isd, v[1] * isd, v[2] * isd, v[3] * isd);
  }
}

// ---------------------------------------------------------------------------------------
// Logits s_h(a) = <q_i^h, k_j^h>/sqrt(d) of the active edges a = (i <- j), one wave per row i.
// q_i is loaded once per row; the row's sources are staged in LDS 128 at a time. Lane = (edge
// slot q of 64/(C/4), channel quad m): each 16-byte load brings 4 channels of k_j, eight
// groups of edges are requested before any is used, and the quads of a head are summed with
// lane swaps. The first lane of each head writes that head's logit.
// ---------------------------------------------------------------------------------------
template <int C, int H>
__global__ void __launch_bounds__(256) k_logits(int32_t n, const int32_t* __restrict__ arow,
                                                const int32_t* __restrict__ asrc,
                                                const float* __restrict__ qk,
                                                float4* __restrict__ es) {
  constexpr int dh = C / H;
  constexpr int CQ = C / 4;     // channel quads
  constexpr int EPG = 64 / CQ;  // edges per group (one per slot)
  constexpr int QH = dh / 4;    // quads per head
  constexpr int kG = 8;         // groups requested together
  static_assert(dh % 4 == 0, "a channel quad must lie in one head");
  __shared__ int32_t sY[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane / CQ, m = lane % CQ;
  const int32_t i = xcd_block(blockIdx.x, gridDim.x) * 4 + wv;
  if (i >= n) return;
  const int hq = (4 * m) / dh;
  const float isd = rsqrtf((float)dh);
  const float4 qv = *reinterpret_cast<const float4*>(qk + (int64_t)i * 2 * C + 4 * m);
  const int32_t a0 = arow[i], a1 = arow[i + 1];
  for (int32_t b = a0; b < a1; b += 128) {
    const int cnt = min(128, a1 - b);
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
      const int l2 = lane + 64 * h2;
      if (l2 < cnt) sY[wv][l2] = asrc[b + l2];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int u = 0; u < cnt; u += kG * EPG) {
      float4 kv[kG];
#pragma unroll
      for (int g = 0; g < kG; g++) {
        const int e = min(u + g * EPG + q, cnt - 1);
        kv[g] = *reinterpret_cast<const float4*>(qk + (int64_t)sY[wv][e] * 2 * C + C + 4 * m);
      }
#pragma unroll
      for (int g = 0; g < kG; g++) {
        float d = qv.x * kv[g].x + qv.y * kv[g].y + qv.z * kv[g].z + qv.w * kv[g].w;
#pragma unroll
        for (int o = 1; o < QH; o <<= 1) d += __shfl_xor(d, o, 64);
        const int e = u + g * EPG + q;
        if (m % QH == 0 && e < cnt) reinterpret_cast<float*>(es)[(int64_t)(b + e) * 4 + hq] = d * isd;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

// ---------------------------------------------------------------------------------------
// Edge contraction on the matrix cores, one wave per row (4 rows per 256-thread block).
//
//   forward (TRANS = false), row = destination i, edges a = (i <- j):
//     M_h = max_a s_ah, Z_h = sum_a u_a exp(s_ah - M_h), alpha_ah = u_a exp(s_ah - M_h)/Z_h,
//     m_i[d3][c] = sum_a alpha_a,h(c) sum_d1 A_a[d3][d1] h_j[d1][c];
//   adjoint (TRANS = true), row = x, edges a = (x <- y) with forward edge e' = rev(a) = (y <- x):
//     hbar_x[d1][c] += alpha_e',h(c) sum_d3 A_e'[d3][d1] mbar_y[d3][c]   (A_e' uses Y(-n_a)).
//
// Chunks of 32 (adjoint: 28) edges: lanes first build alpha and A_e (lane = edge) into
// LDS. The channel sums then run on 4x4x1 MFMA blocks (v_mfma_f32_4x4x1f32: 16 independent
// 4x4 outer products per instruction; block b takes its A column from lanes 4b..4b+3 and
// its B row from the same lanes, and lane 4b+j ends with D_b[r][j] in register r). Lane =
// (edge q of a group of 64/(C/4) edges, channel quad m): it loads 4 consecutive channels of
// one input component with one 16-byte load, and for s = 0..3 feeds channel 4m+s as its A
// value; its B value is the coupling from that input component to output component
// 4g+(lane&3) of the same edge. Blocks of different edges add into separate accumulators
// that are summed over the group's edges once per row. Output components 0..7 use the
// matrix cores (two groups of four), component 8 (l = 2, m = 2) is a vector FMA.
// L0ONLY: only the l = 0 input component is non-zero: the features of the first layer
// (forward; they are the species embedding) or m_bar of the last layer (adjoint).
// ---------------------------------------------------------------------------------------

// OUT0 (forward of the last layer): only output component 0 is formed, on the VALU (each lane
// adds sum_k alpha A_e[0][k] h_j[k][4m..4m+3] for its edge); the energy reads nothing else.
template <int LMAX, int C, int H, bool L0ONLY, bool TRANS, bool OUT0 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((TRANS || L0ONLY || OUT0) ? 4 : 3, 8))) k_edge_contract(
    int32_t n, const int32_t* __restrict__ arow, const float4* __restrict__ ageo,
    const int32_t* __restrict__ asrc, const int32_t* __restrict__ arev,
    const float* __restrict__ ew, const float4* __restrict__ es, const float* __restrict__ X,
    float rc, float* __restrict__ out, const float* __restrict__ base, float4* __restrict__ P,
    const int32_t* __restrict__ species, const float* __restrict__ emb, int S,
    const float* __restrict__ base0, int64_t ews) {
  constexpr int D = Dims<LMAX>::D;
  constexpr int DI = L0ONLY ? 1 : D;          // input components that can be non-zero
  constexpr int CQ = C / 4;                   // channel quads
  constexpr int EPG = 64 / CQ;                // edges per group
  constexpr int NDG = LMAX == 2 ? 2 : 1;      // groups of 4 output components on MFMA
  constexpr bool VC8 = LMAX == 2;             // output component 8 on the VALU
  constexpr int dh = C / H;
  static_assert(C % 16 == 0 && C <= 64 && dh % 4 == 0, "unsupported channel/head split");
  // edges per chunk (the adjoint keeps less in registers and runs 4 waves per SIMD)
  constexpr int kChunk = TRANS ? 28 : 32;
  constexpr int DO = OUT0 ? 1 : D;  // output components formed
  // radial weights that reach the stored coupling entries (the others are neither written
  // for this layer nor read): column 0 only (first layer) -> sender degree 0; row 0 only
  // (last layer's forward and adjoint) -> output degree 0
  constexpr uint32_t WMASK = (L0ONLY && !TRANS) ? paths_from<LMAX>(0)
                             : (OUT0 || (L0ONLY && TRANS)) ? paths_to<LMAX>(0)
                                                          : all_paths<LMAX>();
  __shared__ float sA[4][kChunk][DO * DI];
  __shared__ float sAl[4][kChunk][4];
  __shared__ int32_t sJ[4][kChunk];
  // first layer (forward): the input features are the species embedding (comp 0 only), read
  // from an LDS copy of the table by the source's species instead of gathering the source's row
  constexpr bool EMB = L0ONLY && !TRANS;
  __shared__ float4 sEmb[EMB ? 16 * C / 4 : 1];
  __shared__ int32_t sSp[4][EMB ? kChunk : 1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane / CQ, m = lane % CQ, jj = lane & 3;
  if constexpr (EMB) {
    for (int t = threadIdx.x; t < S * C / 4; t += blockDim.x)
      sEmb[t] = reinterpret_cast<const float4*>(emb)[t];
    __syncthreads();
  }
  const int32_t x = xcd_block(blockIdx.x, gridDim.x) * 4 + wv;
  if (x >= n) return;
  const int32_t a0 = arow[x], a1 = arow[x + 1];
  float Mh[4] = {0.0f, 0.0f, 0.0f, 0.0f}, Zh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!TRANS) {
    // softmax statistics over the row in one pass (lane = edge): each lane keeps its running
    // maximum and its sum of u exp(s - max), rescaled when the maximum grows; lanes are then
    // combined with the wave maximum
    float ml[4], zl[4];
#pragma unroll
    for (int hh = 0; hh < 4; hh++) { ml[hh] = -INFINITY; zl[hh] = 0.0f; }
    for (int32_t a = a0 + lane; a < a1; a += 64) {
      const float4 s4 = es[a];
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
      const float u = 0.5f * (__cosf(kPi * ageo[a].w / rc) + 1.0f);
#pragma unroll
      for (int hh = 0; hh < H; hh++) {
        if (sv[hh] > ml[hh]) {
          zl[hh] = zl[hh] * __expf(ml[hh] - sv[hh]) + u;
          ml[hh] = sv[hh];
        } else {
          zl[hh] += u * __expf(sv[hh] - ml[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < H; hh++) {
      Mh[hh] = wave_max(ml[hh]);
      Zh[hh] = wave_sum(ml[hh] == -INFINITY ? 0.0f : zl[hh] * __expf(ml[hh] - Mh[hh]));
    }
  }
  floatx4 acc[4][NDG];
#pragma unroll
  for (int t = 0; t < 4; t++)
#pragma unroll
    for (int d = 0; d < NDG; d++) acc[t][d] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float4 acc8 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float4 acc0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);  // OUT0
  const int hl = (4 * m) / dh;  // head of this lane's channels
  // Per-edge inputs of a chunk's prologue (lane = edge). The forward requests those of the
  // next chunk before the current chunk's MFMA groups, so their latency is hidden.
  constexpr int PP = Dims<LMAX>::P;
  int32_t pf_y = 0;
  float4 pf_geo = make_float4(0.0f, 0.0f, 0.0f, 1.0f), pf_s4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float pf_w[PP];
  auto prefetch = [&](int32_t bb) {
    const int32_t a = bb + lane;
    if (!TRANS && bb < a1 && lane < min(kChunk, a1 - bb)) {
      pf_y = asrc[a];
      pf_geo = ageo[a];
      pf_s4 = es[a];
#pragma unroll
      for (int p = 0; p < PP; p++) pf_w[p] = ((WMASK >> p) & 1u) ? ew[p * ews + a] : 0.0f;
    }
  };
  prefetch(a0);
  for (int32_t b = a0; b < a1; b += kChunk) {
    const int cnt = min(kChunk, a1 - b);
    if (lane < cnt) {
      const int32_t a = b + lane;
      const int32_t y = TRANS ? asrc[a] : pf_y;
      float4 geo = TRANS ? ageo[a] : pf_geo;
      float u = 0.5f * (__cosf(kPi * geo.w / rc) + 1.0f);
      float sv[4];
      if (!TRANS) {
        // softmax probability p_h = exp(s_h - M_h)/Z_h (kept for the backward), weight u p_h
        float4 s4 = pf_s4;
        sv[0] = s4.x; sv[1] = s4.y; sv[2] = s4.z; sv[3] = s4.w;
        float ph[4];
#pragma unroll
        for (int hh = 0; hh < 4; hh++) {
          ph[hh] = (hh < H && Zh[hh] > 0.0f) ? __expf(sv[hh] - Mh[hh]) / Zh[hh] : 0.0f;
          sAl[wv][lane][hh] = u * ph[hh];
        }
        P[a] = make_float4(ph[0], ph[1], ph[2], ph[3]);
      } else {
        // the forward edge e' = rev(a) = (y <- x): its softmax probability from the forward
        const int32_t ep = arev[a];
        const float4 p4 = P[ep];
        const float ph[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int hh = 0; hh < 4; hh++) sAl[wv][lane][hh] = u * ph[hh];
        (void)sv;
      }
      const float ir = 1.0f / geo.w;
      const float sg = TRANS ? -1.0f : 1.0f;
      float Y[9];
      sph<LMAX>(sg * geo.x * ir, sg * geo.y * ir, sg * geo.z * ir, Y);
      float w[Dims<LMAX>::P];
#pragma unroll
      for (int p = 0; p < Dims<LMAX>::P; p++)
        w[p] = TRANS ? (((WMASK >> p) & 1u) ? ew[p * ews + a] : 0.0f) : pf_w[p];
      float A[D * D];
      coupling_matrix<LMAX>(w, Y, A);
      // row o of the LDS copy lists the coupling of output component o to every input
      // component that can be non-zero: A itself (forward) or its transpose (adjoint); the
      // entries that are never stored are never computed
#pragma unroll
      for (int o = 0; o < DO; o++)
#pragma unroll
        for (int k = 0; k < DI; k++) sA[wv][lane][o * DI + k] = TRANS ? A[k * D + o] : A[o * D + k];
      sJ[wv][lane] = y;
      if constexpr (EMB) sSp[wv][lane] = sp_index(species[y], S);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    prefetch(b + kChunk);
    // Groups of EPG edges; past the chunk's end a lane re-reads the last edge with alpha = 0.
    const int ngroups = (cnt + EPG - 1) / EPG;
    // edge slot of group E for this lane (clamped to the chunk) and its weight alpha
    auto slot = [&](int E, float& ao) {
      const int e0 = E * EPG + q;
      const int e = e0 < cnt ? e0 : cnt - 1;
      ao = e0 < cnt ? sAl[wv][e][hl] : 0.0f;
      return e;
    };
    // alpha depends on (edge, head of the channel). When a head spans 16 channels, the four
    // rows of an MFMA block (channels 16(b%4)+4i+s) share one head, which is also the head of
    // the lane supplying the block's B value, so alpha scales B; otherwise it scales A.
    constexpr bool AL_ON_B = dh % 16 == 0;
    // the contribution of input component k of edge slot e (features xk, weight ai)
    auto mma_k = [&](int k, const float4 xk, float ai, int e) {
      const float* Ae = sA[wv][e];
      if constexpr (OUT0) {
        const float b = ai * Ae[k];
        acc0.x = __builtin_fmaf(b, xk.x, acc0.x);
        acc0.y = __builtin_fmaf(b, xk.y, acc0.y);
        acc0.z = __builtin_fmaf(b, xk.z, acc0.z);
        acc0.w = __builtin_fmaf(b, xk.w, acc0.w);
      } else {
        const float sa = AL_ON_B ? 1.0f : ai;
        const float xs[4] = {sa * xk.x, sa * xk.y, sa * xk.z, sa * xk.w};
#pragma unroll
        for (int d = 0; d < NDG; d++) {
          const float bv = Ae[(4 * d + jj) * DI + k];
          const float bk = AL_ON_B ? ai * bv : bv;
#pragma unroll
          for (int t = 0; t < 4; t++)
            acc[t][d] = __builtin_amdgcn_mfma_f32_4x4x1f32(xs[t], bk, acc[t][d], 0, 0, 0);
        }
        if constexpr (VC8) {
          const float b8 = AL_ON_B ? ai * Ae[8 * DI + k] : Ae[8 * DI + k];
          acc8.x = __builtin_fmaf(b8, xs[0], acc8.x);
          acc8.y = __builtin_fmaf(b8, xs[1], acc8.y);
          acc8.z = __builtin_fmaf(b8, xs[2], acc8.z);
          acc8.w = __builtin_fmaf(b8, xs[3], acc8.w);
        }
      }
    };
    if constexpr (EMB) {
      // first layer: one input component, read from the LDS copy of the embedding
      for (int E = 0; E < ngroups; E++) {
        float al;
        const int e = slot(E, al);
        mma_k(0, sEmb[sSp[wv][e] * (C / 4) + m], al, e);
      }
    } else {
      // Rolling prefetch: each feature register is reloaded with the next group's component
      // as soon as the current group's MFMAs for that component have been issued, so a
      // group's gathers are in flight during the previous group's work without a second
      // register set (the chunk's first group is loaded before the loop).
      float4 xr[DI];
      float al;
      int e = slot(0, al);
      {
        const float* X0 = X + (int64_t)sJ[wv][e] * D * C + 4 * m;
#pragma unroll
        for (int k = 0; k < DI; k++) xr[k] = *reinterpret_cast<const float4*>(X0 + k * C);
      }
      for (int E = 0; E + 1 < ngroups; E++) {
        float aln;
        const int en = slot(E + 1, aln);
        const float* Xn = X + (int64_t)sJ[wv][en] * D * C + 4 * m;
#pragma unroll
        for (int k = 0; k < DI; k++) {
          mma_k(k, xr[k], al, e);
          xr[k] = *reinterpret_cast<const float4*>(Xn + k * C);
        }
        e = en;
        al = aln;
      }
#pragma unroll
      for (int k = 0; k < DI; k++) mma_k(k, xr[k], al, e);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  if constexpr (OUT0) {
#pragma unroll
    for (int o = CQ; o < 64; o <<= 1) {
      acc0.x += __shfl_xor(acc0.x, o, 64);
      acc0.y += __shfl_xor(acc0.y, o, 64);
      acc0.z += __shfl_xor(acc0.z, o, 64);
      acc0.w += __shfl_xor(acc0.w, o, 64);
    }
    if (lane < CQ) *reinterpret_cast<float4*>(out + (int64_t)x * D * C + 4 * m) = acc0;
    return;
  }
  // sum over the edge slots q of a group (lanes CQ apart)
#pragma unroll
  for (int o = CQ; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
      for (int d = 0; d < NDG; d++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc[t][d][r] += __shfl_xor(acc[t][d][r], o, 64);
    if constexpr (VC8) {
      acc8.x += __shfl_xor(acc8.x, o, 64);
      acc8.y += __shfl_xor(acc8.y, o, 64);
      acc8.z += __shfl_xor(acc8.z, o, 64);
      acc8.w += __shfl_xor(acc8.w, o, 64);
    }
  }
  if (lane < CQ) {
    // lane 4bb + jj holds, for tile t and register r, channel 16 bb + 4 r + t of output
    // component 4 d + jj
    // the adjoint adds the residual path: out = base + contribution (every component of
    // every row is written); with base0 set, the base is base0[c] in component 0 and zero in
    // the others (the readout's gradient, for the last layer)
    const int bb = lane >> 2;
    const int64_t ro = (int64_t)x * D * C;
#pragma unroll
    for (int d = 0; d < NDG; d++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t off = ro + (4 * d + jj) * C + 16 * bb + 4 * r;
        float4 v = make_float4(acc[0][d][r], acc[1][d][r], acc[2][d][r], acc[3][d][r]);
        if (TRANS) {
          float4 pv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (!base0)
            pv = *reinterpret_cast<const float4*>(base + off);
          else if (4 * d + jj == 0)
            pv = *reinterpret_cast<const float4*>(base0 + 16 * bb + 4 * r);
          v.x += pv.x; v.y += pv.y; v.z += pv.z; v.w += pv.w;
        }
        *reinterpret_cast<float4*>(out + off) = v;
      }
    if constexpr (VC8) {
      const int64_t off = ro + 8 * C + 4 * m;
      float4 v = acc8;
      if (TRANS && !base0) {
        const float4 pv = *reinterpret_cast<const float4*>(base + off);
        v.x += pv.x; v.y += pv.y; v.z += pv.z; v.w += pv.w;
      }
      *reinterpret_cast<float4*>(out + off) = v;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Adjoints of the attention projections, one wave per row x:
//   qbar_x[c] = sum_a sbar_a,h(c) k_y[c] / sqrt(d)        (x as destination of a = (x <- y)),
//   kbar_x[c] = sum_a sbar_rev(a),h(c) q_y[c] / sqrt(d)   (x as source of rev(a) = (y <- x)).
// The row's per-edge data (neighbour, both logit adjoints) is staged in LDS 128 edges at a
// time (two loads per lane; one stage covers most rows). Lane = (edge slot q of 64/(C/4),
// channel quad m): each 16-byte load covers 4 channels, so one wave request brings whole q|k
// rows of several neighbours. Eight groups of edges are requested before any is used; past
// the row's end a slot repeats the last edge with weight 0. The slots' partial sums are added
// at the end. swapped: sbar of edge e is stored at slot rev(e) (the last layer's edge gradient
// writes it so), and the two reads of each pair exchange.
// ---------------------------------------------------------------------------------------
template <int C, int H>
__global__ void __launch_bounds__(256) k_qk_bar(int32_t n, const int32_t* __restrict__ arow,
                                                const int32_t* __restrict__ asrc,
                                                const int32_t* __restrict__ arev,
                                                const float4* __restrict__ sbar,
                                                const float* __restrict__ qk,
                                                float* __restrict__ qkbar, bool swapped) {
  constexpr int dh = C / H;
  constexpr int CQ = C / 4;     // channel quads
  constexpr int EPG = 64 / CQ;  // edges per group (one per slot)
  constexpr int kG = 8;         // groups requested together
  static_assert(dh % 4 == 0, "a channel quad must lie in one head");
  __shared__ int32_t sY[4][128];
  __shared__ float4 sS[4][128];
  __shared__ float4 sD[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane / CQ, m = lane % CQ;
  const int32_t x = xcd_block(blockIdx.x, gridDim.x) * 4 + wv;
  if (x >= n) return;
  const int hl = (4 * m) / dh;
  float4 qacc = make_float4(0.0f, 0.0f, 0.0f, 0.0f), kacc = qacc;
  const int32_t a0 = arow[x], a1 = arow[x + 1];
  for (int32_t b = a0; b < a1; b += 128) {
    const int cnt = min(128, a1 - b);
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
      const int l2 = lane + 64 * h2;
      if (l2 < cnt) {
        const int32_t e = b + l2;
        sY[wv][l2] = asrc[e];
        const int32_t er = arev[e];
        sS[wv][l2] = sbar[swapped ? e : er];
        sD[wv][l2] = sbar[swapped ? er : e];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int u = 0; u < cnt; u += kG * EPG) {
      float4 qv[kG], kv[kG];
#pragma unroll
      for (int g = 0; g < kG; g++) {
        const int e = min(u + g * EPG + q, cnt - 1);
        const float* row = qk + (int64_t)sY[wv][e] * 2 * C + 4 * m;
        qv[g] = *reinterpret_cast<const float4*>(row);
        kv[g] = *reinterpret_cast<const float4*>(row + C);
      }
#pragma unroll
      for (int g = 0; g < kG; g++) {
        const bool ok = u + g * EPG + q < cnt;
        const int e = min(u + g * EPG + q, cnt - 1);
        const float ss = ok ? reinterpret_cast<const float*>(&sS[wv][e])[hl] : 0.0f;
        const float sd = ok ? reinterpret_cast<const float*>(&sD[wv][e])[hl] : 0.0f;
        kacc.x += ss * qv[g].x; kacc.y += ss * qv[g].y;
        kacc.z += ss * qv[g].z; kacc.w += ss * qv[g].w;
        qacc.x += sd * kv[g].x; qacc.y += sd * kv[g].y;
        qacc.z += sd * kv[g].z; qacc.w += sd * kv[g].w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
#pragma unroll
  for (int o = CQ; o < 64; o <<= 1) {
    qacc.x += __shfl_xor(qacc.x, o, 64); qacc.y += __shfl_xor(qacc.y, o, 64);
    qacc.z += __shfl_xor(qacc.z, o, 64); qacc.w += __shfl_xor(qacc.w, o, 64);
    kacc.x += __shfl_xor(kacc.x, o, 64); kacc.y += __shfl_xor(kacc.y, o, 64);
    kacc.z += __shfl_xor(kacc.z, o, 64); kacc.w += __shfl_xor(kacc.w, o, 64);
  }
  if (lane < CQ) {
    const float isd = rsqrtf((float)dh);
    float* out = qkbar + (int64_t)x * 2 * C + 4 * m;
    *reinterpret_cast<float4*>(out) =
        make_float4(qacc.x * isd, qacc.y * isd, qacc.z * isd, qacc.w * isd);
    *reinterpret_cast<float4*>(out + C) =
        make_float4(kacc.x * isd, kacc.y * isd, kacc.z * isd, kacc.w * isd);
  }
}

// ---------------------------------------------------------------------------------------
// Readout E_i = w_E . h_i^(T, 0) and a deterministic fp64 total.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_readout(int32_t n, int C, int D, const float* __restrict__ h,
                                                 const float* __restrict__ wE,
                                                 float* __restrict__ e_atom,
                                                 double* __restrict__ part) {
  __shared__ double sh[256];
  int32_t i = blockIdx.x * 256 + threadIdx.x;
  double v = 0.0;
  if (i < n) {
    float e = 0.0f;
    for (int c = 0; c < C; c++) e += wE[c] * h[(int64_t)i * D * C + c];
    if (e_atom) e_atom[i] = e;
    v = (double)e;
  }
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

// A non-finite total (some E_i is not finite) sets kStatusNonFinite in the status word.
__global__ void __launch_bounds__(256) k_energy_final(int32_t nb, const double* __restrict__ part,
                                                      double* __restrict__ energy,
                                                      int32_t* __restrict__ status) {
  __shared__ double sh[256];
  double v = 0.0;
  for (int32_t k = threadIdx.x; k < nb; k += 256) v += part[k];
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    energy[0] = sh[0];
    if (!isfinite(sh[0])) atomicOr(status, kStatusNonFinite);
  }
}

// ---------------------------------------------------------------------------------------
// Backward: update adjoint (elementwise part). gbar = dE/dh^(t+1).
//   xcat[n][0:C]      = gbar^0 * SiLU'(y0)
//   xcat[n][lC:(l+1)C] = sum_m gbar^(l,m) y^(l,m) * sigmoid'(g_l)
//   ybl[n][l^2+m][c]  = gbar^(l,m) * sigmoid(g_l)
// (the residual path hbar = gbar + ... is added by the transposed edge contraction)
// MB0 (last layer): only gbar^0 is non-zero and only xcat[n][0:C] is formed (the gates and
// y^(l>=1) of that layer are never computed, so they are not read).
// ---------------------------------------------------------------------------------------
template <int LMAX, bool MB0>
__global__ void k_bwd_update(int32_t n, int C, const float* __restrict__ gbar,
                             const float* __restrict__ yg, const float* __restrict__ yl,
                             float* __restrict__ xcat, float* __restrict__ ybl,
                             const float* __restrict__ wE) {
  constexpr int D = Dims<LMAX>::D;
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (int64_t)n * C) return;
  int64_t i = k / C;
  int c = (int)(k - i * C);
  const int G = C * (1 + LMAX);
  const float* gb = gbar + i * D * C + c;
  float y0 = yg[i * G + c];
  float sg0 = sigmoidf_(y0);
  // wE (last layer): dE/dh^T is the readout's w_E in component 0 (and zero elsewhere)
  xcat[i * G + c] = (wE ? wE[c] : gb[0]) * sg0 * (1.0f + y0 * (1.0f - sg0));
  if constexpr (MB0) return;
#pragma unroll
  for (int l = 1; l <= LMAX; l++) {
    float g = yg[i * G + l * C + c];
    float sg = sigmoidf_(g);
    float s = 0.0f;
    for (int mm = 0; mm < 2 * l + 1; mm++) {
      int d = l * l + mm;
      float gv = gb[d * C];
      s += gv * yl[i * D * C + d * C + c];
      ybl[i * D * C + d * C + c] = gv * sg;
    }
    xcat[i * G + l * C + c] = s * sg * (1.0f - sg);
  }
}

// D_i^h = <mbar_i^h, m_i^h> over the head's channels and all components (MB0: mbar has only
// its l = 0 component). Wave per node.
template <int LMAX, int C, int H, bool MB0>
__global__ void __launch_bounds__(256) k_dst(int32_t n, const float* __restrict__ mbar,
                                             const float* __restrict__ m, float* __restrict__ Dst) {
  constexpr int D = MB0 ? 1 : Dims<LMAX>::D;
  constexpr int DS = Dims<LMAX>::D;  // row stride in components
  constexpr int dh = C / H;
  int32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (i >= n) return;
  float v = 0.0f;
  if (lane < C) {
#pragma unroll
    for (int d = 0; d < D; d++)
      v += mbar[(int64_t)i * DS * C + d * C + lane] * m[(int64_t)i * DS * C + d * C + lane];
  }
#pragma unroll
  for (int o = 1; o < dh; o <<= 1) v += __shfl_xor(v, o, 64);
  if (lane < C && (lane % dh) == 0) Dst[(int64_t)i * H + lane / dh] = v;
}

__global__ void k_gbar_init(int32_t n, int C, int D, const float* __restrict__ wE,
                            float* __restrict__ gbar) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (int64_t)n * D * C) return;
  int rem = (int)(k % (D * C));
  gbar[k] = rem < C ? wE[rem] : 0.0f;
}

// ---------------------------------------------------------------------------------------
// Edge gradient for active edge e = (i <- j), destination-major. One lane per (edge, head):
//   Abar^h = sum_{c in h} mbar_i[:,c] (x) h_j[:,c];  (wbar^h, Ybar^h) = coupling adjoint;
//   abar_h = <A_e, Abar^h> = w . wbar^h;  sbar_h = alpha_h (abar_h - D_ih);
//   ubar = sum_h p_h (abar_h - D_ih), p_h = exp(s_h - M_ih)/Z_ih (stored by the forward
//   contraction), alpha_h = u p_h;
//   wbar = sum_h alpha_h wbar^h, Ybar = sum_h alpha_h Ybar^h  (sums over the edge's lanes);
//   dE/dr = wbar . dw/dr + ubar u'(r);  g = dE/dr n + (I - n n^T) J_Y^T Ybar / r.
// g (dE/dr_vec) accumulates over layers per edge; sbar is kept for the q/k adjoints.
// Each lane reads the head's contiguous channel slice of a feature row of h_j with back-to-back
// 16-byte loads, so the H lanes of an edge together read whole rows; m_bar rows of the
// block's destinations are staged in LDS.
// ---------------------------------------------------------------------------------------
constexpr int kGradRows = 8;    // destination rows of m_bar staged in LDS at a time
constexpr int kGradPasses = 2;  // edges per thread for one staging of m_bar rows

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, false));
}
// Sum over the 4 lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1]); every lane gets it.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  return v;
}

// Coupling adjoint of the rows d1 = L1^2 + S0 .. + NR - 1 of one head's Abar (Ab[d3 NR + m]):
//   t^p[m2] = sum_{m1 in rows, m3} C^p[m1][m2][m3] Abar[(l3,m3)][m1],  wbar^p = t^p . Y_l2;
//   abar += w_p wbar^p;  wb[p] += alpha wbar^p;  Yb[l2^2+m2] += alpha w_p t^p[m2].
// Only the output components d3 < D3N of Abar are read (the others are zero). Used by the
// first and last layers' edge gradients. grad_rows below carries the same loop inline:
// calling this function from it made the compiler spill the full-layer kernel's registers.
template <int LMAX, int L1, int S0, int NR, int D3N, int NA>
__device__ __forceinline__ void grad_adjoint(const float (&Ab)[NA], const float* w,
                                             const float* Y, float al, float& abar, float* wb,
                                             float* Yb) {
  constexpr const CGTable& T = cg_table<LMAX>();
#pragma unroll
  for (int p = 0; p < Dims<LMAX>::P; p++) {
    if (T.l1[p] != L1) continue;
    const float alw = al * w[p];
    float wbh = 0.0f;
    bool touched = false;
#pragma unroll
    for (int m2 = 0; m2 < 5; m2++) {
      if (m2 >= 2 * T.l2[p] + 1) continue;
      float tpm = 0.0f;
      bool any = false;
#pragma unroll
      for (int m = 0; m < NR; m++)
#pragma unroll
        for (int m3 = 0; m3 < 5; m3++) {
          if (m3 < 2 * T.l3[p] + 1 && T.l3[p] * T.l3[p] + m3 < D3N &&
              T.v[p][S0 + m][m2][m3] != 0.0) {
            tpm += (float)T.v[p][S0 + m][m2][m3] * Ab[(T.l3[p] * T.l3[p] + m3) * NR + m];
            any = true;
          }
        }
      if (any) {
        wbh += tpm * Y[T.l2[p] * T.l2[p] + m2];
        Yb[T.l2[p] * T.l2[p] + m2] += alw * tpm;
        touched = true;
      }
    }
    if (touched) {
      abar += w[p] * wbh;
      wb[p] += al * wbh;
    }
  }
}

// Rows d1 = L1^2 + S0 .. L1^2 + S0 + NR - 1 (sender degree L1) of one head's gradient:
// Abar[d3][m1] = sum_{c in head} mbar_i[d3][c] h_j[d1][c] for every output component d3 (all of
// a row's head channels loaded at once), then the part of the coupling adjoint that these
// columns feed (the adjoint is a sum over (d3, d1) entries, so it splits by column; the same
// sums as grad_adjoint).
template <int LMAX, int C, int DH, int L1, int S0, int NR, class MRow>
__device__ __forceinline__ void grad_rows(MRow mrow, const float* __restrict__ h_j, int c0,
                                          const float* w, const float* Y, float al,
                                          float& abar, float* wb, float* Yb) {
  constexpr int D = Dims<LMAX>::D, B0 = L1 * L1 + S0, NC = DH / 4;
  float4 hv[NR][NC];
#pragma unroll
  for (int m = 0; m < NR; m++)
#pragma unroll
    for (int t = 0; t < NC; t++)
      hv[m][t] = *reinterpret_cast<const float4*>(h_j + (B0 + m) * C + c0 + 4 * t);
  float Ab[D * NR];
  float4 mv[NC], mn[NC];
#pragma unroll
  for (int t = 0; t < NC; t++) mv[t] = mrow(c0 + 4 * t);
#pragma unroll
  for (int d3 = 0; d3 < D; d3++) {
    if (d3 + 1 < D) {
#pragma unroll
      for (int t = 0; t < NC; t++) mn[t] = mrow((d3 + 1) * C + c0 + 4 * t);
    }
#pragma unroll
    for (int m = 0; m < NR; m++) {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < NC; t++) {
        acc = __builtin_fmaf(mv[t].x, hv[m][t].x, acc);
        acc = __builtin_fmaf(mv[t].y, hv[m][t].y, acc);
        acc = __builtin_fmaf(mv[t].z, hv[m][t].z, acc);
        acc = __builtin_fmaf(mv[t].w, hv[m][t].w, acc);
      }
      Ab[d3 * NR + m] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NC; t++) mv[t] = mn[t];
  }
  constexpr const CGTable& T = cg_table<LMAX>();
#pragma unroll
  for (int p = 0; p < Dims<LMAX>::P; p++) {
    if (T.l1[p] != L1) continue;
    const float alw = al * w[p];
    float wbh = 0.0f;
    bool touched = false;
#pragma unroll
    for (int m2 = 0; m2 < 5; m2++) {
      if (m2 >= 2 * T.l2[p] + 1) continue;
      float tpm = 0.0f;
      bool any = false;
#pragma unroll
      for (int m = 0; m < NR; m++)
#pragma unroll
        for (int m3 = 0; m3 < 5; m3++) {
          if (m3 < 2 * T.l3[p] + 1 && T.v[p][S0 + m][m2][m3] != 0.0) {
            tpm += (float)T.v[p][S0 + m][m2][m3] * Ab[(T.l3[p] * T.l3[p] + m3) * NR + m];
            any = true;
          }
        }
      if (any) {
        wbh += tpm * Y[T.l2[p] * T.l2[p] + m2];
        Yb[T.l2[p] * T.l2[p] + m2] += alw * tpm;
        touched = true;
      }
    }
    if (touched) {
      abar += w[p] * wbh;
      wb[p] += al * wbh;
    }
  }
}

// All rows of sender degree L1, at most 3 rows at a time.
template <int LMAX, int C, int DH, int L1, class MRow>
__device__ __forceinline__ void grad_block(MRow mrow, const float* __restrict__ h_j, int c0,
                                           const float* w, const float* Y, float al,
                                           float& abar, float* wb, float* Yb) {
  if constexpr (L1 == 0) {
    grad_rows<LMAX, C, DH, 0, 0, 1>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
  } else if constexpr (L1 == 1) {
    grad_rows<LMAX, C, DH, 1, 0, 3>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
  } else {
    grad_rows<LMAX, C, DH, 2, 0, 3>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
    grad_rows<LMAX, C, DH, 2, 3, 2>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
  }
}

template <int LMAX, int C, int H, bool L0ONLY>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) k_edge_grad(const int32_t* __restrict__ arow_n,
                                                   const float4* __restrict__ ageo,
                                                   const int32_t* __restrict__ adst,
                                                   const int32_t* __restrict__ asrc,
                                                   const float* __restrict__ ew,
                                                   const float* __restrict__ edw,
                                                   const float4* __restrict__ prob,
                                                   const float* __restrict__ Dst,
                                                   const float* __restrict__ mbar,
                                                   const float* __restrict__ h, float rc,
                                                   float4* __restrict__ sbar,
                                                   float* __restrict__ gacc, bool accumulate,
                                                   int64_t cap, int64_t ews,
                                                   const int32_t* __restrict__ species,
                                                   const float* __restrict__ emb, int S) {
  static_assert(H == 1 || H == 4, "one lane or a quad of lanes per edge");
  constexpr int D = Dims<LMAX>::D;
  constexpr int P = Dims<LMAX>::P;
  constexpr int dh = C / H;
  constexpr int EPW = 256 / H;               // edges per pass of the block's threads
  constexpr int EPB = kGradPasses * EPW;     // edges per block
  // radial weights this layer reads: the first layer's input has sender degree 0 only
  constexpr uint32_t WMASK = L0ONLY ? paths_from<LMAX>(0) : all_paths<LMAX>();
  __shared__ float4 smb[kGradRows * D * C / 4];
  // first layer: h_j = (e_(s_j), 0, ..., 0) depends on the species only, so
  // Abar^h[d3][0] = sum_{c in h} mbar_i[d3][c] e_s[c] is tabulated per staged row and species
  __shared__ float sU[L0ONLY ? kGradRows * 16 * H * D : 1];
  const int64_t n_act = *arow_n;
  const uint32_t nb_act = (uint32_t)((n_act + EPB - 1) / EPB);
  if (blockIdx.x >= nb_act) return;  // whole block idle
  const int64_t a_base = (int64_t)xcd_block(blockIdx.x, nb_act) * EPB;
  const int hh = (int)threadIdx.x % H;
  // The block's destinations (edges are destination-major) are staged in LDS kGradRows
  // m_bar rows at a time; each edge is processed in the batch that holds its row, and the
  // block's threads take kGradPasses edges each per staged batch.
  const int32_t i_first = adst[a_base];
  const int32_t nrows = adst[min(a_base + (int64_t)EPB, n_act) - 1] - i_first + 1;
  for (int b0 = 0; b0 < nrows; b0 += kGradRows) {
    const int nst = min(nrows - b0, kGradRows);
    if (b0 > 0) __syncthreads();
    {
      const float4* src = reinterpret_cast<const float4*>(mbar + (int64_t)(i_first + b0) * D * C);
      for (int k = threadIdx.x; k < nst * D * C / 4; k += blockDim.x) smb[k] = src[k];
    }
    __syncthreads();
    if constexpr (L0ONLY) {
      // same channel order as the per-edge sum of the other layers
      const float* mf = reinterpret_cast<const float*>(smb);
      for (int k = threadIdx.x; k < nst * S * H * D; k += blockDim.x) {
        const int r = k / (S * H * D), rem = k % (S * H * D);
        const int sp = rem / (H * D), hq = (rem / D) % H, d3 = rem % D;
        const float* mr = mf + (r * D + d3) * C + hq * dh;
        const float* er = emb + sp * C + hq * dh;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < dh; c++) acc = __builtin_fmaf(mr[c], er[c], acc);
        sU[k] = acc;
      }
      __syncthreads();
    }
#pragma unroll 1
  for (int ps = 0; ps < kGradPasses; ps++) {
    const int64_t a = a_base + ps * EPW + threadIdx.x / H;
    const bool active = a < n_act && a < cap;
    const int ri = active ? adst[a] - i_first : -1;
    if (ri < b0 || ri >= b0 + nst) continue;
    const int32_t i = i_first + ri, j = asrc[a];
    const int sj = L0ONLY ? sp_index(species[j], S) : 0;
    float4 g = ageo[a];
    const float r = g.w, ir = 1.0f / r;
    const float nx = g.x * ir, ny = g.y * ir, nz = g.z * ir;
    float th = kPi * r / rc, s1, c1;
    __sincosf(th, &s1, &c1);
    const float u = 0.5f * (c1 + 1.0f), du = -0.5f * (kPi / rc) * s1;
    float Y[9];
    sph<LMAX>(nx, ny, nz, Y);
    float w[P];
#pragma unroll
    for (int p = 0; p < P; p++) w[p] = ((WMASK >> p) & 1u) ? ew[p * ews + a] : 0.0f;
    float wb[P], Yb[9];
#pragma unroll
    for (int p = 0; p < P; p++) wb[p] = 0.0f;
#pragma unroll
    for (int d = 0; d < 9; d++) Yb[d] = 0.0f;
    const float* h_j = h + (int64_t)j * D * C;
    const int lbase = (ri - b0) * (D * C / 4);
    auto mrow = [&](int off) { return smb[lbase + (off >> 2)]; };
    const float p_h = reinterpret_cast<const float*>(prob)[a * 4 + hh];
    const float al = u * p_h;
    float abar = 0.0f;
    const int c0 = hh * dh;
    if constexpr (L0ONLY) {
      const float* u0 = sU + (((ri - b0) * S + sj) * H + hh) * D;
      float Ab[D];
#pragma unroll
      for (int d3 = 0; d3 < D; d3++) Ab[d3] = u0[d3];
      grad_adjoint<LMAX, 0, 0, 1, D>(Ab, w, Y, al, abar, wb, Yb);
      (void)h_j;
      (void)mrow;
    } else {
      grad_block<LMAX, C, dh, 0>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
      grad_block<LMAX, C, dh, 1>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
      if constexpr (LMAX >= 2) grad_block<LMAX, C, dh, 2>(mrow, h_j, c0, w, Y, al, abar, wb, Yb);
    }
    const float diff = abar - Dst[(int64_t)i * H + hh];
    const float sb = al * diff;
    float ubar = p_h * diff;
    if constexpr (H == 4) {  // sums over the heads of this edge
#pragma unroll
      for (int p = 0; p < P; p++) wb[p] = quad_sum(wb[p]);
#pragma unroll
      for (int d = 0; d < 9; d++) Yb[d] = quad_sum(Yb[d]);
      ubar = quad_sum(ubar);
      reinterpret_cast<float*>(sbar)[a * 4 + hh] = sb;
    } else {
      sbar[a] = make_float4(sb, 0.0f, 0.0f, 0.0f);
    }
    if (hh == 0) {
      float dEdr = ubar * du;
#pragma unroll
      for (int p = 0; p < P; p++)
        if ((WMASK >> p) & 1u) dEdr += wb[p] * edw[p * ews + a];
      float gy[3];
      sph_vjp<LMAX>(nx, ny, nz, Yb, gy);
      const float ng = nx * gy[0] + ny * gy[1] + nz * gy[2];
      float gx = dEdr * nx + (gy[0] - ng * nx) * ir;
      float gyv = dEdr * ny + (gy[1] - ng * ny) * ir;
      float gz = dEdr * nz + (gy[2] - ng * nz) * ir;
      if (accumulate) {
        gx += gacc[a * 3]; gyv += gacc[a * 3 + 1]; gz += gacc[a * 3 + 2];
      }
      gacc[a * 3] = gx;
      gacc[a * 3 + 1] = gyv;
      gacc[a * 3 + 2] = gz;
    }
  }
  }
}

// Edge gradient of the last layer, source-major. There m_bar has only its l = 0 component, so
// Abar^h[0][d1] = sum_{c in h} mbar_i[0][c] h_j[d1][c] needs a full feature row only of the
// source j. The lanes walk the active list grouped by row j (entry a' = (j <- i)) and
// compute the gradient of the forward edge e = rev(a') = (i <- j): h_j rows are staged in LDS
// per block and only mbar_i's l = 0 head slice (64 B per lane) is gathered, instead of the
// 2.3 KB of h_j per edge of the destination-major form. The geometry of e is -r_vec(a') and
// its radial weights are those of a' (both bit-exact, |r| is the same); the softmax
// probability and D_i are read at e. The outputs are written at a' = rev(e), so that the lanes'
// stores are consecutive: sbar_e goes to slot a' (the q/k adjoints of this layer read the two
// slots of each pair the other way round), and -g_e is added to slot a' of the per-edge
// gradient sum. The forces use that sum only as g_a - g_rev(a) per pair, which is unchanged.
// The per-edge sums run in the same order as in k_edge_grad, so sbar and g are identical to its
// single-row form.
template <int LMAX, int C, int H>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) k_edge_grad_last(
    const int32_t* __restrict__ arow_n, const float4* __restrict__ ageo,
    const int32_t* __restrict__ adst, const int32_t* __restrict__ asrc,
    const int32_t* __restrict__ arev, const float* __restrict__ ew, const float* __restrict__ edw,
    const float4* __restrict__ prob, const float* __restrict__ Dst,
    const float* __restrict__ mbar, const float* __restrict__ h, float rc,
    float4* __restrict__ sbar, float* __restrict__ gacc, bool accumulate, int64_t cap,
    int64_t ews) {
  static_assert(H == 1 || H == 4, "one lane or a quad of lanes per edge");
  constexpr int D = Dims<LMAX>::D;
  constexpr int P = Dims<LMAX>::P;
  constexpr int dh = C / H;
  constexpr int NC = dh / 4;
  constexpr int EPW = 256 / H;
  constexpr int EPB = kGradPasses * EPW;
  // radial weights of the paths into output degree 0 (m_bar has only its l = 0 component)
  constexpr uint32_t WMASK = paths_to<LMAX>(0);
  __shared__ float4 shj[kGradRows * D * C / 4];
  const int64_t n_act = *arow_n;
  const uint32_t nb_act = (uint32_t)((n_act + EPB - 1) / EPB);
  if (blockIdx.x >= nb_act) return;
  const int64_t a_base = (int64_t)xcd_block(blockIdx.x, nb_act) * EPB;
  const int hh = (int)threadIdx.x % H;
  const int32_t j_first = adst[a_base];
  const int32_t nrows = adst[min(a_base + (int64_t)EPB, n_act) - 1] - j_first + 1;
  for (int b0 = 0; b0 < nrows; b0 += kGradRows) {
    const int nst = min(nrows - b0, kGradRows);
    if (b0 > 0) __syncthreads();
    {
      const float4* src = reinterpret_cast<const float4*>(h + (int64_t)(j_first + b0) * D * C);
      for (int k = threadIdx.x; k < nst * D * C / 4; k += blockDim.x) shj[k] = src[k];
    }
    __syncthreads();
#pragma unroll 1
    for (int ps = 0; ps < kGradPasses; ps++) {
      const int64_t a = a_base + ps * EPW + threadIdx.x / H;  // a' = (j <- i)
      const bool active = a < n_act && a < cap;
      const int rj = active ? adst[a] - j_first : -1;
      if (rj < b0 || rj >= b0 + nst) continue;
      const int32_t i = asrc[a];
      const int64_t e = arev[a];  // e = (i <- j)
      const float4 g = ageo[a];
      const float r = g.w, ir = 1.0f / r;
      const float nx = -g.x * ir, ny = -g.y * ir, nz = -g.z * ir;
      float th = kPi * r / rc, s1, c1;
      __sincosf(th, &s1, &c1);
      const float u = 0.5f * (c1 + 1.0f), du = -0.5f * (kPi / rc) * s1;
      float Y[9];
      sph<LMAX>(nx, ny, nz, Y);
      float w[P];
#pragma unroll
      for (int p = 0; p < P; p++) w[p] = ((WMASK >> p) & 1u) ? ew[p * ews + a] : 0.0f;
      float wb[P], Yb[9];
#pragma unroll
      for (int p = 0; p < P; p++) wb[p] = 0.0f;
#pragma unroll
      for (int d = 0; d < 9; d++) Yb[d] = 0.0f;
      const float p_h = reinterpret_cast<const float*>(prob)[e * 4 + hh];
      const float al = u * p_h;
      const int c0 = hh * dh;
      // mbar_i[0][head channels]
      float4 mv[NC];
#pragma unroll
      for (int t = 0; t < NC; t++)
        mv[t] = *reinterpret_cast<const float4*>(mbar + (int64_t)i * D * C + c0 + 4 * t);
      const float4* hrow = shj + (rj - b0) * (D * C / 4) + c0 / 4;
      float Ab[D];
#pragma unroll
      for (int d1 = 0; d1 < D; d1++) {
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < NC; t++) {
          const float4 hv = hrow[d1 * (C / 4) + t];
          acc = __builtin_fmaf(mv[t].x, hv.x, acc);
          acc = __builtin_fmaf(mv[t].y, hv.y, acc);
          acc = __builtin_fmaf(mv[t].z, hv.z, acc);
          acc = __builtin_fmaf(mv[t].w, hv.w, acc);
        }
        Ab[d1] = acc;
      }
      float abar = 0.0f;
      {  // the same row blocks, in the same order, as the destination-major kernel
        const float a0[1] = {Ab[0]};
        grad_adjoint<LMAX, 0, 0, 1, 1>(a0, w, Y, al, abar, wb, Yb);
        if constexpr (LMAX >= 1) {
          const float a1[3] = {Ab[1], Ab[2], Ab[3]};
          grad_adjoint<LMAX, 1, 0, 3, 1>(a1, w, Y, al, abar, wb, Yb);
        }
        if constexpr (LMAX >= 2) {
          const float a2[3] = {Ab[4], Ab[5], Ab[6]};
          grad_adjoint<LMAX, 2, 0, 3, 1>(a2, w, Y, al, abar, wb, Yb);
          const float a3[2] = {Ab[7], Ab[8]};
          grad_adjoint<LMAX, 2, 3, 2, 1>(a3, w, Y, al, abar, wb, Yb);
        }
      }
      const float diff = abar - Dst[(int64_t)i * H + hh];
      const float sb = al * diff;
      float ubar = p_h * diff;
      if constexpr (H == 4) {
#pragma unroll
        for (int p = 0; p < P; p++) wb[p] = quad_sum(wb[p]);
#pragma unroll
        for (int d = 0; d < 9; d++) Yb[d] = quad_sum(Yb[d]);
        ubar = quad_sum(ubar);
        reinterpret_cast<float*>(sbar)[a * 4 + hh] = sb;
      } else {
        sbar[a] = make_float4(sb, 0.0f, 0.0f, 0.0f);
      }
      if (hh == 0) {
        float dEdr = ubar * du;
#pragma unroll
        for (int p = 0; p < P; p++)
          if ((WMASK >> p) & 1u) dEdr += wb[p] * edw[p * ews + a];
        float gy[3];
        sph_vjp<LMAX>(nx, ny, nz, Yb, gy);
        const float ng = nx * gy[0] + ny * gy[1] + nz * gy[2];
        float gx = dEdr * nx + (gy[0] - ng * nx) * ir;
        float gyv = dEdr * ny + (gy[1] - ng * ny) * ir;
        float gz = dEdr * nz + (gy[2] - ng * nz) * ir;
        float b0x = 0.0f, b0y = 0.0f, b0z = 0.0f;
        if (accumulate) {
          b0x = gacc[a * 3]; b0y = gacc[a * 3 + 1]; b0z = gacc[a * 3 + 2];
        }
        gacc[a * 3] = b0x - gx;
        gacc[a * 3 + 1] = b0y - gyv;
        gacc[a * 3 + 2] = b0z - gz;
      }
    }
  }
}

// F_x = sum over the row's active edges a of (g_a - g_rev(a)); one wave per row, lanes over
// edges, a fixed-order wave sum (deterministic). A non-finite force sets kStatusNonFinite.
__global__ void __launch_bounds__(256) k_forces(int32_t n, const int32_t* __restrict__ arow,
                                                const int32_t* __restrict__ arev,
                                                const float* __restrict__ gacc,
                                                float* __restrict__ F,
                                                int32_t* __restrict__ status) {
  const int32_t x = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (x >= n) return;
  float f0 = 0.0f, f1 = 0.0f, f2 = 0.0f;
  for (int32_t a = arow[x] + lane; a < arow[x + 1]; a += 64) {
    const int32_t b = arev[a];
    f0 += gacc[(int64_t)a * 3] - gacc[(int64_t)b * 3];
    f1 += gacc[(int64_t)a * 3 + 1] - gacc[(int64_t)b * 3 + 1];
    f2 += gacc[(int64_t)a * 3 + 2] - gacc[(int64_t)b * 3 + 2];
  }
  f0 = wave_sum(f0);
  f1 = wave_sum(f1);
  f2 = wave_sum(f2);
  if (lane == 0) {
    F[3 * (int64_t)x] = f0;
    F[3 * (int64_t)x + 1] = f1;
    F[3 * (int64_t)x + 2] = f2;
    if (!(isfinite(f0) && isfinite(f1) && isfinite(f2))) atomicOr(status, kStatusNonFinite);
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Workspace of the energy/force pass.
// ---------------------------------------------------------------------------------------
struct EFWS {
  float *WqkT, *W0T, *WlT;  // per layer transposed weights
  float *h, *qk, *m, *yg, *yl;
  int32_t *arow, *adst, *asrc, *aslot, *slot2act, *arev, *rev_own;
  float4* ageo;
  float* ar;  // |r| of each active edge (a copy of ageo's w, read 4 edges per 16-byte load)
  float *ew, *edw;
  float4* es;
  float4* P;  // per layer and active edge: softmax probability of each head
  float *gbar, *hbar, *mbar, *xcat, *ybl, *qkbar, *Dst, *gacc;
  float4* sbar;
  float4* l0tab;  // first layer: logits of every (destination species, source species) pair
  float* rtab;    // per layer: radial weights and their r-derivatives at the table's knots
  uint32_t* rchk;  // per layer: the table guard's deviations and scales (float bits)
  double* epart;
  int32_t* scan_tmp;
};

// Row stride of the path-major radial-weight arrays: the edge capacity rounded up to 64.
inline int64_t ews_of(int64_t ecap) { return (ecap + 63) & ~int64_t(63); }

static EFWS carve_ef(Carver& cv, const tess_model_desc& md, int32_t n, int64_t cap) {
  EFWS w{};
  const int64_t C = md.channels, Lm = md.l_max, T = md.n_layers, H = md.n_heads;
  const int64_t D = (Lm + 1) * (Lm + 1);
  const int64_t nn = n > 0 ? n : 1, ec = cap > 0 ? cap : 1;
  w.WqkT = cv.take<float>(T * C * 2 * C);
  w.W0T = cv.take<float>(T * C * C * (1 + Lm));
  w.WlT = cv.take<float>(T * Lm * C * C + 1);
  w.h = cv.take<float>((T + 1) * nn * D * C);
  w.qk = cv.take<float>(T * nn * 2 * C);
  w.m = cv.take<float>(T * nn * D * C);
  w.yg = cv.take<float>(T * nn * C * (1 + Lm));
  w.yl = cv.take<float>(T * nn * D * C);
  w.arow = cv.take<int32_t>(nn + 1);
  w.adst = cv.take<int32_t>(ec);
  w.asrc = cv.take<int32_t>(ec);
  w.aslot = cv.take<int32_t>(ec);
  w.slot2act = cv.take<int32_t>(ec);
  w.arev = cv.take<int32_t>(ec);
  w.rev_own = cv.take<int32_t>(ec);
  w.ageo = cv.take<float4>(ec);
  w.ar = cv.take<float>(ews_of(ec));
  w.ew = cv.take<float>(T * ews_of(ec) * 12);
  w.edw = cv.take<float>(T * ews_of(ec) * 12);
  w.es = cv.take<float4>(T * ec);
  w.P = cv.take<float4>(T * ec);
  w.gbar = cv.take<float>(nn * D * C);
  w.hbar = cv.take<float>(nn * D * C);
  w.mbar = cv.take<float>(nn * D * C);
  w.xcat = cv.take<float>(nn * C * (1 + Lm));
  w.ybl = cv.take<float>(nn * D * C);
  w.qkbar = cv.take<float>(nn * 2 * C);
  w.Dst = cv.take<float>(nn * H);
  w.gacc = cv.take<float>(ec * 3);
  w.sbar = cv.take<float4>(ec);
  w.l0tab = cv.take<float4>(16 * 16);
  w.rtab = cv.take<float>(T * (kRadKnots + 1) * 24);
  w.rchk = cv.take<uint32_t>(4 * T);
  w.epart = cv.take<double>(nn / 256 + 2);
  w.scan_tmp = cv.take<int32_t>(nn / 4096 + 4);
  return w;
}

int64_t ef_workspace_bytes(const tess_model_desc& md, int32_t n, int64_t cap) {
  Carver cv{nullptr, 0};
  carve_ef(cv, md, n, cap);
  return cv.off;
}

namespace {

struct LayerW {
  const float *Wq, *Wk, *W1, *W2, *W0, *Wl[3];
};

// A second stream per host thread and device for kernels of the pass that do not depend on
// the work next to them: the radial-weight table needs only the weights and is built next to
// the active-edge list; layer t+1's q|k GEMM and logits need only the l = 0 features that
// layer t's first update GEMM writes, and run next to that layer's l >= 1 updates; in the
// backward, the l = 0 block of m_bar runs next to the l >= 1 blocks. The stream forks from
// and joins the caller's stream through events, so the caller sees one stream-ordered pass
// and the fork/join become graph edges under stream capture. Created on first use; if it
// cannot be created (or the first call comes under capture), every kernel runs on the
// caller's stream in the same order.
constexpr int kEvFwdFork = 0, kEvFwdJoin = 1, kEvBwdFork = 2, kEvBwdJoin = 3, kEvTabFork = 4,
              kEvTabDone = 5, kEvChkDone = 6, kAuxEvents = 7;
struct AuxStream {
  bool tried = false, ok = false;
  hipStream_t s = nullptr;
  hipEvent_t ev[kAuxEvents] = {};
};
AuxStream* aux_stream(hipStream_t st) {
  constexpr int kMaxDev = 16;
  thread_local AuxStream a[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return nullptr;
  }
  AuxStream& x = a[dev];
  if (!x.tried) {
    // the stream is created outside any stream capture (a capture in progress runs the pass
    // on the caller's stream alone; a later call outside capture creates it)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (cs != hipStreamCaptureStatusNone) return nullptr;
    x.tried = true;
    bool ok = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess;
    for (int k = 0; k < kAuxEvents && ok; k++)
      ok = hipEventCreateWithFlags(&x.ev[k], hipEventDisableTiming) == hipSuccess;
    x.ok = ok;
    if (!ok) (void)hipGetLastError();
  }
  return x.ok ? &x : nullptr;
}
// `to` waits for everything enqueued so far on `from` (through event k of the pool).
inline hipError_t stream_after(AuxStream* ax, int k, hipStream_t from, hipStream_t to) {
  hipError_t e = hipEventRecord(ax->ev[k], from);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(to, ax->ev[k], 0);
}

template <int LMAX, int C, int H, int R>
int32_t ef_run(const tess_model_desc& md, const float* weights, int32_t n, const float box[3],
               const float* pos, const int32_t* species, const int32_t* row_ptr,
               const uint32_t* col_shift, const int32_t* rev_in, int64_t n_edges, int64_t ecap,
               double* energy, float* e_atom, float* forces, const EFWS& w, int32_t* status,
               hipStream_t st, uint32_t* rmin2_bits) {
  constexpr int D = Dims<LMAX>::D;
  constexpr int P = Dims<LMAX>::P;
  constexpr int G = C * (1 + LMAX);
  const int T = md.n_layers, S = md.n_species, K = md.n_rbf;
  const float rc = md.r_cut;
  const int64_t cap = n_edges > 0 ? n_edges : 0;  // threads per edge kernel
  const int64_t ews = ews_of(ecap > 0 ? ecap : 1);  // row stride of the radial-weight arrays
  // ecap: edge capacity the workspace was laid out for (strides of per-layer edge arrays)
  // weight offsets in the blob
  std::vector<LayerW> lw(T);
  {
    int64_t off = (int64_t)S * C;
    for (int t = 0; t < T; t++) {
      lw[t].Wq = weights + off; off += C * C;
      lw[t].Wk = weights + off; off += C * C;
      lw[t].W1 = weights + off; off += (int64_t)R * K;
      lw[t].W2 = weights + off; off += (int64_t)P * R;
      lw[t].W0 = weights + off; off += (int64_t)G * C;
      for (int l = 1; l <= LMAX; l++) { lw[t].Wl[l] = weights + off; off += C * C; }
    }
  }
  const float* emb = weights;
  const float* wE = weights + (int64_t)S * C + (int64_t)T * (2 * C * C + R * K + P * R + G * C + LMAX * C * C);
  // transposed weights
  {
    constexpr int NEL = 2 * C * C + G * C + LMAX * C * C;
    k_prep_weights<LMAX, C, R><<<dim3(gridn(NEL, 256), T), 256, 0, st>>>(weights, S, K, w.WqkT,
                                                                         w.W0T, w.WlT);
  }
  // The library's second stream (see aux_stream).
  AuxStream* ax = aux_stream(st);
  const hipStream_t sb = ax ? ax->s : st;
  // radial-weight table of every layer: it depends on the weights only and runs on the second
  // stream next to the active-edge list (joined before the interpolation)
  if (ax) TESS_HIP_CHECK(stream_after(ax, kEvTabFork, st, sb));
  const int64_t lstride = (int64_t)(2 * C * C + R * K + P * R + G * C + LMAX * C * C);
  k_radial_table<P><<<dim3(gridn(kRadKnots + 1, 256), T), 256, 0, sb>>>(lw[0].W1, lstride, R,
                                                                        rc, w.rtab);
  TESS_HIP_CHECK(hipGetLastError());
  if (ax) TESS_HIP_CHECK(hipEventRecord(ax->ev[kEvTabDone], sb));
  // the table's guard runs behind it on the same stream, next to the forward pass (joined
  // before the energy is summed)
  k_fill_i32<<<1, 64, 0, sb>>>(reinterpret_cast<int32_t*>(w.rchk), 4 * T, 0);
  k_radial_check<P><<<dim3(gridn(kRadKnots, 256), T), 256, 0, sb>>>(lw[0].W1, lstride, R, rc,
                                                                    w.rtab, w.rchk);
  k_radial_verdict<<<1, 64, 0, sb>>>(T, w.rchk, status);
  TESS_HIP_CHECK(hipGetLastError());
  if (ax) TESS_HIP_CHECK(hipEventRecord(ax->ev[kEvChkDone], sb));
  const int64_t NDC = (int64_t)n * D * C;
  // embedding
  k_embed<<<gridn((int64_t)n * C, 256), 256, 0, st>>>(n, C, D, S, species, emb, w.h, status);
  // active edges
  const int32_t* rev = rev_in;
  if (cap > 0) {
    if (!rev) {
      // reverse index: each pair searched once in its target row (rows are sorted)
      TESS_HIP_CHECK(rev_index(n, row_ptr, col_shift, w.rev_own, st));
      rev = w.rev_own;
    }
    k_active_count<<<gridn(n, 4), 256, 0, st>>>(n, pos, row_ptr, col_shift, box[0], box[1], box[2],
                                                rc * rc, w.arow, rmin2_bits);
    TESS_HIP_CHECK(scan_exclusive_i32(w.arow, (int64_t)n + 1, w.scan_tmp, st));
    k_active_fill<<<gridn(n, 4), 256, 0, st>>>(n, pos, row_ptr, col_shift, box[0], box[1], box[2],
                                               rc * rc, w.arow, w.adst, w.asrc, w.aslot,
                                               w.slot2act, w.ageo, w.ar);
    k_active_rev<<<gridn(cap, 256), 256, 0, st>>>(w.arow + n, w.aslot, rev, w.slot2act, w.arev, cap);
    TESS_HIP_CHECK(hipGetLastError());
  } else {
    k_fill_i32<<<gridn((int64_t)n + 1, 256), 256, 0, st>>>(w.arow, (int64_t)n + 1, 0);
  }
  const RowMap feat0{(int64_t)D * C, C, 0, 1};
  // q|k GEMM and logits of layer t (t >= 1) on stream `qs`
  auto qk_logits = [&](int t, hipStream_t qs) -> int32_t {
    Epi e0{};
    e0.y = w.qk + (int64_t)t * n * 2 * C;
    e0.ym = RowMap{2 * C, 0, 0, 1};
    TESS_HIP_CHECK(gemm<EPI_STORE>(qs, n, C, 2 * C, w.h + (int64_t)t * NDC, feat0,
                                   w.WqkT + (int64_t)t * C * 2 * C, e0));
    if (cap > 0)
      TESS_TIMED("logits", qs,
                 k_logits<C, H><<<gridn(n, 4), 256, 0, qs>>>(n, w.arow, w.asrc, e0.y,
                                                            w.es + (int64_t)t * ecap));
    TESS_HIP_CHECK(hipGetLastError());
    return TESS_OK;
  };
  // first layer: logits from the per-species table (q and k of the first layer are not needed
  // anywhere else: the backward stops before dE/dh^0); then the radial weights of every layer
  // and the first layer's logits for each active edge
  k_l0_logits<C, H><<<1, 256, 0, st>>>(S, emb, lw[0].Wq, lw[0].Wk, w.l0tab);
  if (ax) TESS_HIP_CHECK(hipStreamWaitEvent(st, ax->ev[kEvTabDone], 0));
  if (cap > 0)
    TESS_TIMED("edge_radial", st,
               k_edge_radial<P><<<kRadBlocks, kRadThreads, 0, st>>>(
                   w.arow + n, w.ar, w.rtab, 0, T, rc, w.ew, w.edw, ews * 12, ews, cap,
                   w.adst, w.asrc, species, w.l0tab, S, w.es, paths_from<LMAX>(0),
                   paths_to<LMAX>(0)));
  TESS_HIP_CHECK(hipGetLastError());
  // ---------------- forward ----------------
  for (int t = 0; t < T; t++) {
    float* ht = w.h + (int64_t)t * NDC;
    float* hn = w.h + (int64_t)(t + 1) * NDC;
    float4* Pt = w.P + (int64_t)t * ecap;
    float* mt = w.m + (int64_t)t * NDC;
    float* yg = w.yg + (int64_t)t * n * G;
    float* yl = w.yl + (int64_t)t * NDC;
    float* ew = w.ew + (int64_t)t * ews * 12;
    float4* es = w.es + (int64_t)t * ecap;
    if (t > 0) {
      if (ax) {
        // q|k and logits were enqueued on the third stream after the previous layer's l = 0
        // update
        TESS_HIP_CHECK(hipStreamWaitEvent(st, ax->ev[kEvFwdJoin], 0));
      } else {
        const int32_t rq = qk_logits(t, st);
        if (rq != TESS_OK) return rq;
      }
    }
    if (t == 0)
      TESS_TIMED("edge_apply", st,
                 k_edge_contract<LMAX, C, H, true, false><<<gridn(n, 4), 256, 0, st>>>(
                     n, w.arow, w.ageo, w.asrc, w.arev, ew, es, ht, rc, mt, nullptr, Pt, species,
                     emb, S, nullptr, ews));
    else if (t == T - 1)  // last layer: only m^0 is read (by the y^0 update)
      TESS_TIMED("edge_apply", st,
                 k_edge_contract<LMAX, C, H, false, false, true><<<gridn(n, 4), 256, 0, st>>>(
                     n, w.arow, w.ageo, w.asrc, w.arev, ew, es, ht, rc, mt, nullptr, Pt, species,
                     emb, S, nullptr, ews));
    else
      TESS_TIMED("edge_apply", st,
                 k_edge_contract<LMAX, C, H, false, false><<<gridn(n, 4), 256, 0, st>>>(
                     n, w.arow, w.ageo, w.asrc, w.arev, ew, es, ht, rc, mt, nullptr, Pt, species,
                     emb, S, nullptr, ews));
    TESS_HIP_CHECK(hipGetLastError());
    Epi eu{};
    eu.y = yg;
    eu.ym = RowMap{G, 0, 0, 1};
    eu.hin = ht;
    eu.hout = hn;
    eu.hm = feat0;
    eu.cdim = C;
    // last layer (when not also the first): the energy reads only h^T's l = 0 channels, so
    // neither the gates nor the l >= 1 updates are formed (the backward of that layer reads
    // only y^0)
    const bool last = t == T - 1 && t > 0;
    TESS_HIP_CHECK(gemm<EPI_UPD0>(st, n, C, G, mt, feat0, w.W0T + (int64_t)t * C * G, eu,
                                  last ? C : 0));
    if (ax && t + 1 < T) {
      // the next layer's q|k and logits read only h^(t+1)'s l = 0 block, written above
      TESS_HIP_CHECK(stream_after(ax, kEvFwdFork, st, sb));
      const int32_t rq = qk_logits(t + 1, sb);
      if (rq != TESS_OK) return rq;
      TESS_HIP_CHECK(hipEventRecord(ax->ev[kEvFwdJoin], sb));
    }
    for (int l = 1; l <= LMAX && !last; l++) {
      RowMap ml{(int64_t)D * C, C, l * l, 2 * l + 1};
      Epi el{};
      el.y = yl;
      el.ym = ml;
      el.hin = t == 0 ? nullptr : ht;  // h^0 has no l >= 1 components
      el.hout = hn;
      el.hm = ml;
      el.gates = yg;
      el.gstride = G;
      el.goff = l * C;
      el.cdim = C;
      TESS_HIP_CHECK(gemm<EPI_UPDL>(st, (int64_t)n * (2 * l + 1), C, C, mt, ml,
                                    w.WlT + ((int64_t)t * LMAX + (l - 1)) * C * C, el));
    }
  }
  // readout
  const float* hT = w.h + (int64_t)T * NDC;
  int32_t nb = gridn(n, 256);
  if (nb > 0) k_readout<<<nb, 256, 0, st>>>(n, C, D, hT, wE, e_atom, w.epart);
  if (ax) TESS_HIP_CHECK(hipStreamWaitEvent(st, ax->ev[kEvChkDone], 0));
  k_energy_final<<<1, 256, 0, st>>>(nb, w.epart, energy, status);
  TESS_HIP_CHECK(hipGetLastError());
  if (!forces) return TESS_OK;
  // ---------------- backward ----------------
  float* gbar = w.gbar;
  float* hbar = w.hbar;
  // dE/dh^T: w_E in the l = 0 channels. With more than one layer, the last layer's kernels
  // read w_E directly (only its l = 0 part is non-zero); a single layer reads the buffer.
  if (T == 1) k_gbar_init<<<gridn(NDC, 256), 256, 0, st>>>(n, C, D, wE, gbar);
  for (int t = T - 1; t >= 0; t--) {
    const float* ht = w.h + (int64_t)t * NDC;
    const float* qk = w.qk + (int64_t)t * n * 2 * C;
    float4* Pt = w.P + (int64_t)t * ecap;
    const float* mt = w.m + (int64_t)t * NDC;
    const float* yg = w.yg + (int64_t)t * n * G;
    const float* yl = w.yl + (int64_t)t * NDC;
    const float* ew = w.ew + (int64_t)t * ews * 12;
    const float* edw = w.edw + (int64_t)t * ews * 12;
    const float4* es = w.es + (int64_t)t * ecap;
    const bool mb0 = t == T - 1 && t > 0;
    if (mb0)
      k_bwd_update<LMAX, true><<<gridn((int64_t)n * C, 256), 256, 0, st>>>(n, C, gbar, yg, yl,
                                                                         w.xcat, w.ybl, wE);
    else
      k_bwd_update<LMAX, false><<<gridn((int64_t)n * C, 256), 256, 0, st>>>(
          n, C, gbar, yg, yl, w.xcat, w.ybl, nullptr);
    // The energy reads only the l = 0 channels of the last features, so at the last layer
    // dE/dh^(l>=1) = 0: the gate adjoints and the l >= 1 components of m_bar vanish. That layer
    // (when it is not also the first) forms only m_bar's l = 0 component and its edge kernels
    // use only that component (the other components of the buffer are never read).
    Epi em{};
    em.y = w.mbar;
    em.ym = feat0;
    // the l = 0 block of m_bar and the l >= 1 blocks read and write disjoint data
    const bool fork = ax && !mb0;
    const hipStream_t s0 = fork ? sb : st;
    if (fork) TESS_HIP_CHECK(stream_after(ax, kEvBwdFork, st, sb));
    TESS_HIP_CHECK(gemm<EPI_STORE>(s0, n, mb0 ? C : G, C, w.xcat, RowMap{G, 0, 0, 1}, lw[t].W0,
                                   em));
    if (fork) TESS_HIP_CHECK(hipEventRecord(ax->ev[kEvBwdJoin], sb));
    for (int l = 1; l <= LMAX && !mb0; l++) {
      RowMap ml{(int64_t)D * C, C, l * l, 2 * l + 1};
      Epi el{};
      el.y = w.mbar;
      el.ym = ml;
      TESS_HIP_CHECK(gemm<EPI_STORE>(st, (int64_t)n * (2 * l + 1), C, C, w.ybl, ml, lw[t].Wl[l], el));
    }
    if (fork) TESS_HIP_CHECK(hipStreamWaitEvent(st, ax->ev[kEvBwdJoin], 0));
    if (mb0)
      k_dst<LMAX, C, H, true><<<gridn(n, 4), 256, 0, st>>>(n, w.mbar, mt, w.Dst);
    else
      k_dst<LMAX, C, H, false><<<gridn(n, 4), 256, 0, st>>>(n, w.mbar, mt, w.Dst);
    if (cap > 0) {
      const int32_t gb = gridn(cap, kGradPasses * 256 / H);
      if (t == 0)
        TESS_TIMED("edge_grad", st,
                   k_edge_grad<LMAX, C, H, true><<<gb, 256, 0, st>>>(
                       w.arow + n, w.ageo, w.adst, w.asrc, ew, edw, Pt, w.Dst, w.mbar, ht, rc,
                       w.sbar, w.gacc, t != T - 1, cap, ews, species, emb, S));
      else if (mb0)
        TESS_TIMED("edge_grad_last", st,
                   k_edge_grad_last<LMAX, C, H><<<gb, 256, 0, st>>>(
                       w.arow + n, w.ageo, w.adst, w.asrc, w.arev, ew, edw, Pt, w.Dst, w.mbar, ht,
                       rc, w.sbar, w.gacc, t != T - 1, cap, ews));
      else
        TESS_TIMED("edge_grad", st,
                   k_edge_grad<LMAX, C, H, false><<<gb, 256, 0, st>>>(
                       w.arow + n, w.ageo, w.adst, w.asrc, ew, edw, Pt, w.Dst, w.mbar, ht, rc,
                       w.sbar, w.gacc, t != T - 1, cap, ews, species, emb, S));
    }
    TESS_HIP_CHECK(hipGetLastError());
    if (t > 0) {
      if (mb0)  // only m_bar's l = 0 component enters the adjoint contraction; the residual
                // input is the readout's gradient w_E in component 0
        TESS_TIMED("edge_tapply", st,
                   k_edge_contract<LMAX, C, H, true, true><<<gridn(n, 4), 256, 0, st>>>(
                       n, w.arow, w.ageo, w.asrc, w.arev, ew, es, w.mbar, rc, hbar, nullptr, Pt,
                       species, emb, S, wE, ews));
      else
        TESS_TIMED("edge_tapply", st,
                   k_edge_contract<LMAX, C, H, false, true><<<gridn(n, 4), 256, 0, st>>>(
                       n, w.arow, w.ageo, w.asrc, w.arev, ew, es, w.mbar, rc, hbar, gbar, Pt,
                       species, emb, S, nullptr, ews));
      // the last layer's source-major edge gradient stores sbar of edge e at slot rev(e)
      k_qk_bar<C, H><<<gridn(n, 4), 256, 0, st>>>(n, w.arow, w.asrc, w.arev, w.sbar, qk,
                                                 w.qkbar, mb0);
      Epi ea{};
      ea.y = hbar;
      ea.ym = feat0;
      TESS_HIP_CHECK(gemm<EPI_ADD>(st, n, 2 * C, C, w.qkbar, RowMap{2 * C, 0, 0, 1}, lw[t].Wq, ea));
      float* tmp = gbar;
      gbar = hbar;
      hbar = tmp;
    }
  }
  if (cap > 0) {
    k_forces<<<gridn(n, 4), 256, 0, st>>>(n, w.arow, w.arev, w.gacc, forces, status);
  } else if (n > 0) {
    k_fill_f32<<<gridn(3 * (int64_t)n, 256), 256, 0, st>>>(forces, 3 * (int64_t)n, 0.0f);
  }
  TESS_HIP_CHECK(hipGetLastError());
  return TESS_OK;
}

}  // namespace

bool ef_shape_supported(const tess_model_desc& md) {
  if (md.n_rbf != 8 || md.n_layers < 1 || md.n_layers > 16 || md.n_species < 1 ||
      md.n_species > 16 || !(md.r_cut > 0.0f))
    return false;
  const int l = md.l_max, c = md.channels, h = md.n_heads, r = md.radial_hidden;
  return (l == 1 && c == 16 && h == 1 && r == 32) || (l == 2 && c == 32 && h == 4 && r == 32) ||
         (l == 2 && c == 64 && h == 4 && r == 64) || (l == 2 && c == 16 && h == 4 && r == 32) ||
         (l == 1 && c == 32 && h == 4 && r == 32);
}

int32_t ef_dispatch(const tess_model_desc& md, const float* weights, int32_t n, const float box[3],
                    const float* pos, const int32_t* species, const int32_t* row_ptr,
                    const uint32_t* col_shift, const int32_t* rev, int64_t n_edges,
                    int64_t ecap, double* energy, float* e_atom, float* forces, char* ws,
                    int64_t ws_bytes, int32_t* status, hipStream_t st, uint32_t* rmin2_bits) {
  Carver cv{ws, 0};
  EFWS w = carve_ef(cv, md, n, ecap);
  if (cv.off > ws_bytes) return TESS_ERR_WORKSPACE;
  const int l = md.l_max, c = md.channels, h = md.n_heads, r = md.radial_hidden;
#define TESS_EF_CASE(L_, C_, H_, R_)                                                          \
  if (l == L_ && c == C_ && h == H_ && r == R_)                                               \
    return ef_run<L_, C_, H_, R_>(md, weights, n, box, pos, species, row_ptr, col_shift, rev, \
                                  n_edges, ecap, energy, e_atom, forces, w, status, st,       \
                                  rmin2_bits);
  TESS_EF_CASE(1, 16, 1, 32)
  TESS_EF_CASE(2, 32, 4, 32)
  TESS_EF_CASE(2, 64, 4, 64)
  TESS_EF_CASE(2, 16, 4, 32)
  TESS_EF_CASE(1, 32, 4, 32)
#undef TESS_EF_CASE
  return TESS_ERR_ARG;
}

}  // namespace tess
