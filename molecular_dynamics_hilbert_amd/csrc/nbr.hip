// nbr.hip -- neighbour-list rebuild on gfx950.
//
// The three levels of the Tessera abstract's neighbour search (space-filling-curve order,
// cells, pair filter with a conservative skin), as four stages:
//   1. wrap + 30-bit Hilbert key per atom (fp64, every operation rounded on its own),
//   2. stable LSD radix sort of (key, index), 4 passes of 8 bits; each 1024-key tile ranks
//      its keys with wave ballots (64 lanes) so equal digits keep their index order,
//   3. cell binning (cells at least (r_cut+skin)(1+1e-6) wide),
//   4. per atom one wave scans the 27 neighbouring cells; the fp64 pair test decides, the
//      wave compacts passing pairs with ballot + popcount, and a bitonic sort in LDS puts each
//      row in ascending (j, shift) order. Count pass, scan, fill pass.
// Decisions that must match the fp64 reference bit for bit are written with FP contraction
// off.
#include "tess_common.h"

#pragma clang fp contract(off)

namespace tess {
namespace {

constexpr int kMaxRow = 1024;
constexpr int kTile = 1024;  // radix-sort tile (256 threads x 4 rounds)

__device__ __forceinline__ float wrap_coord(float x, double L) {
  double t = (double)x / L;
  double f = floor(t);
  double p = f * L;
  double xw = (double)x - p;
  return (float)xw;
}

__device__ __forceinline__ uint32_t quant10(float xw, double L) {
  double S = 1024.0 / L;
  double v = floor((double)xw * S);
  v = v < 0.0 ? 0.0 : (v > 1023.0 ? 1023.0 : v);
  return (uint32_t)v;
}

// Skilling's transpose-form Hilbert index for 3 axes, 10 bits per axis; key bits are read
// level by level (most significant first), axis 0 first within a level.
__device__ __forceinline__ uint32_t hilbert30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t X[3] = {x0, x1, x2};
#pragma unroll
  for (uint32_t Q = 1u << 9; Q > 1; Q >>= 1) {
    uint32_t P = Q - 1;
#pragma unroll
    for (int i = 0; i < 3; i++) {
      if (X[i] & Q) {
        X[0] ^= P;
      } else {
        uint32_t t = (X[0] ^ X[i]) & P;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];
  X[2] ^= X[1];
  uint32_t t = 0;
#pragma unroll
  for (uint32_t Q = 1u << 9; Q > 1; Q >>= 1)
    if (X[2] & Q) t ^= Q - 1;
  X[0] ^= t; X[1] ^= t; X[2] ^= t;
  uint32_t key = 0;
#pragma unroll
  for (int lev = 9; lev >= 0; lev--)
    key = (key << 3) | (((X[0] >> lev) & 1u) << 2) | (((X[1] >> lev) & 1u) << 1) |
          ((X[2] >> lev) & 1u);
  return key;
}

// Morton (Z-order) key of the same quantised cell: bits interleaved level by level, axis 0
// most significant within a level. Used only when a comparison run selects it.
__device__ __forceinline__ uint32_t morton30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t key = 0;
#pragma unroll
  for (int lev = 9; lev >= 0; lev--)
    key = (key << 3) | (((x0 >> lev) & 1u) << 2) | (((x1 >> lev) & 1u) << 1) | ((x2 >> lev) & 1u);
  return key;
}

__global__ void k_wrap_key(int32_t n, int curve, double Lx, double Ly, double Lz,
                           const float* __restrict__ pos,
                           const int32_t* __restrict__ species, const float* __restrict__ vel,
                           const float* __restrict__ forces, const int32_t* __restrict__ pa,
                           float* __restrict__ pos_w, uint32_t* __restrict__ key,
                           int32_t* __restrict__ idx, int32_t* __restrict__ sp_tmp,
                           float* __restrict__ v_tmp, float* __restrict__ f_tmp,
                           int32_t* __restrict__ pa_tmp) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float x = wrap_coord(pos[3 * i + 0], Lx);
  float y = wrap_coord(pos[3 * i + 1], Ly);
  float z = wrap_coord(pos[3 * i + 2], Lz);
  pos_w[3 * i + 0] = x;
  pos_w[3 * i + 1] = y;
  pos_w[3 * i + 2] = z;
  const uint32_t q0 = quant10(x, Lx), q1 = quant10(y, Ly), q2 = quant10(z, Lz);
  key[i] = curve == 1 ? morton30(q0, q1, q2) : hilbert30(q0, q1, q2);
  idx[i] = i;
  sp_tmp[i] = species[i];
  if (vel)
    for (int a = 0; a < 3; a++) v_tmp[3 * i + a] = vel[3 * i + a];
  if (forces)
    for (int a = 0; a < 3; a++) f_tmp[3 * i + a] = forces[3 * i + a];
  if (pa) pa_tmp[i] = pa[i];
}

__global__ void __launch_bounds__(256) k_radix_hist(const uint32_t* __restrict__ keys, int32_t n,
                                                    int shift, int32_t* __restrict__ hist,
                                                    int32_t nblk) {
  __shared__ int32_t cnt[256];
  int t = threadIdx.x;
  cnt[t] = 0;
  __syncthreads();
  int64_t base = (int64_t)blockIdx.x * kTile;
  for (int r = 0; r < kTile / 256; r++) {
    int64_t i = base + r * 256 + t;
    if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[(int64_t)t * nblk + blockIdx.x] = cnt[t];
}

// Stable scatter of one 8-bit digit. Items are visited in index order (round, wave, lane);
// within a wave the rank among equal digits comes from 8 ballots.
__global__ void __launch_bounds__(256) k_radix_scatter(const uint32_t* __restrict__ kin,
                                                       const int32_t* __restrict__ vin,
                                                       uint32_t* __restrict__ kout,
                                                       int32_t* __restrict__ vout, int32_t n,
                                                       int shift, const int32_t* __restrict__ hist,
                                                       int32_t nblk) {
  __shared__ int32_t base_off[256];
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[4][256];
  int t = threadIdx.x, w = t >> 6, lane = t & 63;
  base_off[t] = hist[(int64_t)t * nblk + blockIdx.x];
  run[t] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int64_t base = (int64_t)blockIdx.x * kTile;
  for (int r = 0; r < kTile / 256; r++) {
#pragma unroll
    for (int ww = 0; ww < 4; ww++) wcnt[ww][t] = 0;
    __syncthreads();
    int64_t i = base + r * 256 + t;
    bool valid = i < n;
    uint32_t key = valid ? kin[i] : 0u;
    uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
      bool bit = (d >> b) & 1u;
      uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    int rank = __popcll(peers & lt);
    if (valid && rank == 0) wcnt[w][d] = __popcll(peers);
    __syncthreads();
    {
      int acc = run[t];
#pragma unroll
      for (int ww = 0; ww < 4; ww++) {
        int c = wcnt[ww][t];
        wcnt[ww][t] = acc;
        acc += c;
      }
      run[t] = acc;
    }
    __syncthreads();
    if (valid) {
      int64_t p = (int64_t)base_off[d] + wcnt[w][d] + rank;
      kout[p] = key;
      vout[p] = vin[i];
    }
    __syncthreads();
  }
}

__global__ void k_permute(int32_t n, const int32_t* __restrict__ idx, const uint32_t* __restrict__ key,
                          const float* __restrict__ pos_w, const int32_t* __restrict__ sp_tmp,
                          const float* __restrict__ v_tmp, const float* __restrict__ f_tmp,
                          const int32_t* __restrict__ pa_tmp, float* __restrict__ pos,
                          int32_t* __restrict__ species, float* __restrict__ vel,
                          float* __restrict__ forces, int32_t* __restrict__ pa,
                          float* __restrict__ ref_pos, int32_t* __restrict__ perm,
                          uint32_t* __restrict__ hkey) {
  int32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  int32_t o = idx[k];
  float x = pos_w[3 * o], y = pos_w[3 * o + 1], z = pos_w[3 * o + 2];
  pos[3 * k] = x; pos[3 * k + 1] = y; pos[3 * k + 2] = z;
  if (ref_pos) { ref_pos[3 * k] = x; ref_pos[3 * k + 1] = y; ref_pos[3 * k + 2] = z; }
  species[k] = sp_tmp[o];
  if (vel)
    for (int a = 0; a < 3; a++) vel[3 * k + a] = v_tmp[3 * o + a];
  if (forces)
    for (int a = 0; a < 3; a++) forces[3 * k + a] = f_tmp[3 * o + a];
  if (pa) pa[k] = pa_tmp[o];
  perm[k] = o;
  if (hkey) hkey[k] = key[k];
}

struct CellGrid {
  int nc[3];
  double L[3];
};

__device__ __forceinline__ int cell_coord(float x, int nc, double L) {
  int v = (int)floor((double)x * (double)nc / L);
  return v < 0 ? 0 : (v >= nc ? nc - 1 : v);
}

__global__ void k_cell_count(int32_t n, CellGrid g, const float* __restrict__ pos,
                             int32_t* __restrict__ cell_id, int32_t* __restrict__ cnt) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int cx = cell_coord(pos[3 * i], g.nc[0], g.L[0]);
  int cy = cell_coord(pos[3 * i + 1], g.nc[1], g.L[1]);
  int cz = cell_coord(pos[3 * i + 2], g.nc[2], g.L[2]);
  int c = (cx * g.nc[1] + cy) * g.nc[2] + cz;
  cell_id[i] = c;
  atomicAdd(&cnt[c], 1);
}

__global__ void k_cell_fill(int32_t n, const int32_t* __restrict__ cell_id,
                            const int32_t* __restrict__ cell_start, int32_t* __restrict__ fill,
                            int32_t* __restrict__ atoms) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int c = cell_id[i];
  int slot = atomicAdd(&fill[c], 1);
  atoms[cell_start[c] + slot] = i;
}

// One wave (one 64-thread block) per atom. FILL = false counts, FILL = true writes the
// sorted row.
template <bool FILL>
__global__ void __launch_bounds__(64) k_pairs(int32_t n, CellGrid g, double rcs2,
                                              const float* __restrict__ pos,
                                              const int32_t* __restrict__ cell_id,
                                              const int32_t* __restrict__ cell_start,
                                              const int32_t* __restrict__ cell_atoms,
                                              int32_t* __restrict__ row_ptr,
                                              uint32_t* __restrict__ col_shift,
                                              int32_t* __restrict__ misc) {
  __shared__ int32_t vstart[27], vcode[27], vpre[28];
  __shared__ uint32_t buf[FILL ? kMaxRow : 1];
  (void)n;  // one block per atom: the grid is n blocks
  if constexpr (FILL) (void)misc;
  const int32_t i = blockIdx.x;
  const int lane = threadIdx.x;
  const double xi0 = (double)pos[3 * i], xi1 = (double)pos[3 * i + 1], xi2 = (double)pos[3 * i + 2];
  int32_t csize = 0;
  if (lane < 27) {
    int c = cell_id[i];
    int cz = c % g.nc[2], cy = (c / g.nc[2]) % g.nc[1], cx = c / (g.nc[1] * g.nc[2]);
    int d[3] = {lane / 9 - 1, (lane / 3) % 3 - 1, lane % 3 - 1};
    int cc[3] = {cx + d[0], cy + d[1], cz + d[2]};
    int s[3];
    for (int a = 0; a < 3; a++) {
      s[a] = 0;
      if (cc[a] < 0) { cc[a] += g.nc[a]; s[a] = -1; }
      else if (cc[a] >= g.nc[a]) { cc[a] -= g.nc[a]; s[a] = 1; }
    }
    int cell = (cc[0] * g.nc[1] + cc[1]) * g.nc[2] + cc[2];
    const int32_t c0 = cell_start[cell];
    vstart[lane] = c0;
    vcode[lane] = 9 * (s[0] + 1) + 3 * (s[1] + 1) + (s[2] + 1);
    csize = cell_start[cell + 1] - c0;
  }
  // inclusive prefix of the 27 cell sizes across lanes (wave scan), vpre[v] = start of cell v
  {
    int32_t inc = csize;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < 27) vpre[lane + 1] = inc;
    if (lane == 0) vpre[0] = 0;
  }
  __syncthreads();
  const int total = vpre[27];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int count = 0;
  // Candidates q0 + lane and q0 + 64 + lane are tested together (two independent load
  // chains per lane); their ballots are consumed in candidate order.
  for (int q0 = 0; q0 < total; q0 += 128) {
    bool pass[2] = {false, false};
    uint32_t entry[2] = {0u, 0u};
    int32_t jv[2];
    int vv[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int q = q0 + 64 * h + lane;
      ok[h] = q < total;
      int lo = 0, hi = 27;  // find v with vpre[v] <= q < vpre[v+1]
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (vpre[mid] <= q) lo = mid; else hi = mid;
      }
      vv[h] = lo;
      jv[h] = ok[h] ? cell_atoms[vstart[lo] + (q - vpre[lo])] : i;
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int32_t j = jv[h];
      const int code = vcode[vv[h]];
      double s0 = (double)(code / 9 - 1), s1 = (double)((code / 3) % 3 - 1),
             s2 = (double)(code % 3 - 1);
      double r0 = ((double)pos[3 * j] - xi0) + s0 * g.L[0];
      double r1 = ((double)pos[3 * j + 1] - xi1) + s1 * g.L[1];
      double r2 = ((double)pos[3 * j + 2] - xi2) + s2 * g.L[2];
      double rr = r0 * r0 + r1 * r1;
      rr = rr + r2 * r2;
      pass[h] = ok[h] && (rr < rcs2) && !(j == i && code == 13);
      entry[h] = ((uint32_t)j << 5) | (uint32_t)code;
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      uint64_t m = __ballot(pass[h]);
      if (FILL) {
        int slot = count + __popcll(m & lt);
        if (pass[h] && slot < kMaxRow) buf[slot] = entry[h];
      }
      count += __popcll(m);
    }
  }
  if (!FILL) {
    if (lane == 0) row_ptr[i] = count;
    return;
  }
  if (count > kMaxRow) return;  // rejected on the host before this pass runs
  int64_t o = row_ptr[i];
  __syncthreads();
  if (count <= 256) {
    // rank sort: keys within a row are distinct, so an entry's position is the number of
    // smaller keys (the wave reads every key once, a broadcast LDS read per key)
    uint32_t mine[4];
    int rank[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      mine[u] = lane + 64 * u < count ? buf[lane + 64 * u] : 0xFFFFFFFFu;
      rank[u] = 0;
    }
    for (int k = 0; k < count; k++) {
      const uint32_t y = buf[k];
#pragma unroll
      for (int u = 0; u < 4; u++) rank[u] += y < mine[u] ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
      if (lane + 64 * u < count)
        col_shift[o + rank[u]] = (mine[u] >> 5) | ((mine[u] & 31u) << 27);
    return;
  }
  int p2 = 1;
  while (p2 < count) p2 <<= 1;
  for (int k = count + lane; k < p2; k += 64) buf[k] = 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = lane; t < (p2 >> 1); t += 64) {
        int a = 2 * jj * (t / jj) + (t % jj);
        int b = a + jj;
        uint32_t va = buf[a], vb = buf[b];
        bool up = (a & k) == 0;
        if ((va > vb) == up) { buf[a] = vb; buf[b] = va; }
      }
      __syncthreads();
    }
  }
  for (int k = lane; k < count; k += 64) {
    uint32_t e = buf[k];
    col_shift[o + k] = (e >> 5) | ((e & 31u) << 27);
  }
}

// Longest row and total pair count of a scanned CSR: block reductions, one atomic of each
// per block. The scan adds in 32 bits, so a total beyond the int32 range of row_ptr wraps
// there; each row's count is still the difference of its (wrapped) bounds, and their 64-bit
// sum is the true total.
__global__ void __launch_bounds__(256) k_max_row(int32_t n, const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ out,
                                                 unsigned long long* __restrict__ total) {
  int32_t i = blockIdx.x * 256 + threadIdx.x;
  int v = i < n ? (int)((uint32_t)row_ptr[i + 1] - (uint32_t)row_ptr[i]) : 0;
  unsigned long long s = (unsigned long long)v;
  for (int o = 32; o >= 1; o >>= 1) {
    v = max(v, __shfl_xor(v, o, 64));
    s += __shfl_xor(s, o, 64);
  }
  __shared__ int32_t sh[4];
  __shared__ unsigned long long ss[4];
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = v;
    ss[threadIdx.x >> 6] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicMax(out, max(max(sh[0], sh[1]), max(sh[2], sh[3])));
    atomicAdd(total, ss[0] + ss[1] + ss[2] + ss[3]);
  }
}

// rev[e] for every pair of row i: position of (j <- i, 26 - code) in row j (rows are sorted
// by (j, code)). One wave per row.
__global__ void __launch_bounds__(256) k_rev(int32_t n, const int32_t* __restrict__ row_ptr,
                                             const uint32_t* __restrict__ col,
                                             int32_t* __restrict__ rev) {
  int32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (i >= n) return;
  int32_t b = row_ptr[i], e_end = row_ptr[i + 1];
  // two entries per lane, their binary searches interleaved (independent load chains)
  for (int32_t e0 = b + lane; e0 < e_end; e0 += 128) {
    int32_t lo[2], hi[2];
    uint32_t want[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int32_t e = e0 + 64 * h;
      ok[h] = e < e_end;
      const uint32_t c = col[ok[h] ? e : e0];
      const int32_t j = (int32_t)(c & 0x7FFFFFFu);
      want[h] = ((uint32_t)i << 5) | (26u - (c >> 27));
      lo[h] = ok[h] ? row_ptr[j] : 0;
      hi[h] = ok[h] ? row_ptr[j + 1] : 0;
    }
    while (lo[0] < hi[0] || lo[1] < hi[1]) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (lo[h] < hi[h]) {
          const int32_t mid = (lo[h] + hi[h]) >> 1;
          const uint32_t cm = col[mid];
          const uint32_t km = ((cm & 0x7FFFFFFu) << 5) | (cm >> 27);
          if (km < want[h]) lo[h] = mid + 1; else hi[h] = mid;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (ok[h]) rev[e0 + 64 * h] = lo[h];
  }
}

// ---- scan -----------------------------------------------------------------------------
constexpr int kScanTile = 4096;  // 256 threads x 16

__device__ __forceinline__ int32_t block_exclusive_scan_256(int32_t v, int32_t* sh, int32_t* total) {
  int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    if (k < w) off += sh[k];
    tot += sh[k];
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Two arrays of the same length can be scanned by the same launches: blockIdx.y (partial,
// final) or blockIdx.x (sums) selects the array, and its tile sums sit nb entries apart.
struct ScanPair {
  int32_t* d[2];
};

__global__ void __launch_bounds__(256) k_scan_partial(ScanPair sp, int64_t n,
                                                      int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  const int32_t* __restrict__ d = sp.d[blockIdx.y];
  int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int32_t s = 0;
  for (int k = 0; k < 16; k++)
    if (base + k < n) s += d[base + k];
  int32_t tot;
  block_exclusive_scan_256(s, sh, &tot);
  if (threadIdx.x == 0) sums[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = tot;
}

__global__ void __launch_bounds__(256) k_scan_sums(int32_t* __restrict__ sums_all, int32_t nb) {
  __shared__ int32_t sh[4];
  int32_t* __restrict__ sums = sums_all + (int64_t)blockIdx.x * nb;
  int32_t carry = 0;
  for (int32_t b0 = 0; b0 < nb; b0 += 256) {
    int32_t k = b0 + threadIdx.x;
    int32_t v = k < nb ? sums[k] : 0;
    int32_t tot;
    int32_t ex = block_exclusive_scan_256(v, sh, &tot);
    if (k < nb) sums[k] = carry + ex;
    carry += tot;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) k_scan_final(ScanPair sp, int64_t n,
                                                    const int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  int32_t* __restrict__ d = sp.d[blockIdx.y];
  int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int32_t v[16];
  int32_t s = 0;
  for (int k = 0; k < 16; k++) {
    v[k] = (base + k < n) ? d[base + k] : 0;
    s += v[k];
  }
  int32_t tot;
  int32_t run = block_exclusive_scan_256(s, sh, &tot) +
                sums[(int64_t)blockIdx.y * gridDim.x + blockIdx.x];
  for (int k = 0; k < 16; k++) {
    if (base + k < n) d[base + k] = run;
    run += v[k];
  }
}

inline int32_t grid(int64_t n, int b) { return (int32_t)((n + b - 1) / b); }

}  // namespace

hipError_t scan_exclusive_i32(int32_t* data, int64_t n, int32_t* partial, hipStream_t s) {
  return scan_exclusive_i32_pair(data, nullptr, n, partial, s);
}

hipError_t scan_exclusive_i32_pair(int32_t* a, int32_t* b, int64_t n, int32_t* partial,
                                   hipStream_t s) {
  int32_t nb = grid(n, kScanTile);
  if (nb == 0) return hipSuccess;
  const unsigned na = b ? 2u : 1u;
  ScanPair sp{{a, b ? b : a}};
  k_scan_partial<<<dim3(nb, na), 256, 0, s>>>(sp, n, partial);
  k_scan_sums<<<na, 256, 0, s>>>(partial, nb);
  k_scan_final<<<dim3(nb, na), 256, 0, s>>>(sp, n, partial);
  return hipGetLastError();
}

hipError_t rev_index(int32_t n, const int32_t* row_ptr, const uint32_t* col, int32_t* rev,
                     hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_rev<<<grid(n, 4), 256, 0, s>>>(n, row_ptr, col, rev);
  return hipGetLastError();
}

NbrWS carve_nbr(Carver& c, int32_t n) {
  NbrWS w{};
  int64_t nn = n > 0 ? n : 1;
  int64_t nblk = (nn + kTile - 1) / kTile;
  w.ncell_cap = 2 * nn + 64;
  w.pos_w = c.take<float>(3 * nn);
  w.key[0] = c.take<uint32_t>(nn);
  w.key[1] = c.take<uint32_t>(nn);
  w.idx[0] = c.take<int32_t>(nn);
  w.idx[1] = c.take<int32_t>(nn);
  w.hist = c.take<int32_t>(256 * nblk + 1);
  w.sp_tmp = c.take<int32_t>(nn);
  w.pa_tmp = c.take<int32_t>(nn);
  w.v_tmp = c.take<float>(3 * nn);
  w.f_tmp = c.take<float>(3 * nn);
  w.cell_start = c.take<int32_t>(w.ncell_cap + 1);
  w.cell_fill = c.take<int32_t>(w.ncell_cap);
  w.cell_atoms = c.take<int32_t>(nn);
  w.cell_id = c.take<int32_t>(nn);
  int64_t scan_len = (256 * nblk + 1 > w.ncell_cap + 1 ? 256 * nblk + 1 : w.ncell_cap + 1);
  if (nn + 1 > scan_len) scan_len = nn + 1;
  w.scan_tmp = c.take<int32_t>(scan_len / kScanTile + 2);
  w.misc = c.take<int32_t>(16);
  return w;
}

int32_t build_neighbors_impl(int32_t n, const float box[3], float r_cut, float skin, float* pos,
                             int32_t* species, float* vel, float* ref_pos, float* forces,
                             int32_t* perm_accum, int32_t* perm, uint32_t* hkey,
                             int32_t* row_ptr, uint32_t* col_shift, int32_t* rev,
                             int64_t edge_cap, int64_t* n_edges, const NbrWS& ws,
                             hipStream_t st) {
  const double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  const double rcs = (double)r_cut + (double)skin;
  const double rcs2 = rcs * rcs;
  // 1. wrap + keys
  k_wrap_key<<<grid(n, 256), 256, 0, st>>>(n, sort_curve(), L[0], L[1], L[2], pos, species,
                                           vel, forces,
                                           perm_accum, ws.pos_w, ws.key[0], ws.idx[0], ws.sp_tmp,
                                           ws.v_tmp, ws.f_tmp, ws.pa_tmp);
  TESS_HIP_CHECK(hipGetLastError());
  // 2. stable radix sort, 4 x 8 bits (keys have 30 bits)
  int32_t nblk = grid(n, kTile);
  int cur = 0;
  for (int pass = 0; pass < 4; pass++) {
    int shift = 8 * pass;
    k_radix_hist<<<nblk, 256, 0, st>>>(ws.key[cur], n, shift, ws.hist, nblk);
    TESS_HIP_CHECK(scan_exclusive_i32(ws.hist, (int64_t)256 * nblk, ws.scan_tmp, st));
    TESS_TIMED("radix_scatter", st,
               k_radix_scatter<<<nblk, 256, 0, st>>>(ws.key[cur], ws.idx[cur], ws.key[cur ^ 1],
                                                     ws.idx[cur ^ 1], n, shift, ws.hist, nblk));
    TESS_HIP_CHECK(hipGetLastError());
    cur ^= 1;
  }
  // permute every per-atom array into sorted order
  k_permute<<<grid(n, 256), 256, 0, st>>>(n, ws.idx[cur], ws.key[cur], ws.pos_w, ws.sp_tmp,
                                          vel ? ws.v_tmp : nullptr, forces ? ws.f_tmp : nullptr,
                                          perm_accum ? ws.pa_tmp : nullptr, pos, species, vel,
                                          forces, perm_accum, ref_pos, perm, hkey);
  TESS_HIP_CHECK(hipGetLastError());
  // 3. cells
  CellGrid g;
  int64_t ncell = 1;
  for (int a = 0; a < 3; a++) {
    g.L[a] = L[a];
    int k = (int)floor(L[a] / (rcs * (1.0 + 1e-6)));
    g.nc[a] = k < 1 ? 1 : k;
  }
  for (;;) {
    ncell = (int64_t)g.nc[0] * g.nc[1] * g.nc[2];
    if (ncell <= ws.ncell_cap) break;
    int a = (g.nc[0] >= g.nc[1] && g.nc[0] >= g.nc[2]) ? 0 : (g.nc[1] >= g.nc[2] ? 1 : 2);
    g.nc[a]--;
  }
  TESS_HIP_CHECK(hipMemsetAsync(ws.cell_start, 0, sizeof(int32_t) * (ncell + 1), st));
  TESS_HIP_CHECK(hipMemsetAsync(ws.cell_fill, 0, sizeof(int32_t) * ncell, st));
  TESS_HIP_CHECK(hipMemsetAsync(ws.misc, 0, sizeof(int32_t) * 16, st));
  k_cell_count<<<grid(n, 256), 256, 0, st>>>(n, g, pos, ws.cell_id, ws.cell_start);
  TESS_HIP_CHECK(scan_exclusive_i32(ws.cell_start, ncell + 1, ws.scan_tmp, st));
  k_cell_fill<<<grid(n, 256), 256, 0, st>>>(n, ws.cell_id, ws.cell_start, ws.cell_fill,
                                            ws.cell_atoms);
  TESS_HIP_CHECK(hipGetLastError());
  // 4. pairs: count, scan, check, fill
  TESS_HIP_CHECK(hipMemsetAsync(row_ptr + n, 0, sizeof(int32_t), st));
  TESS_TIMED("nbr_count", st,
             k_pairs<false><<<n, 64, 0, st>>>(n, g, rcs2, pos, ws.cell_id, ws.cell_start,
                                              ws.cell_atoms, row_ptr, nullptr, ws.misc));
  TESS_HIP_CHECK(hipGetLastError());
  TESS_HIP_CHECK(scan_exclusive_i32(row_ptr, (int64_t)n + 1, ws.scan_tmp, st));
  // misc[0]: longest row; misc[4..5]: 64-bit pair total (the block is 256-byte aligned)
  unsigned long long* total = reinterpret_cast<unsigned long long*>(ws.misc + 4);
  k_max_row<<<grid(n, 256), 256, 0, st>>>(n, row_ptr, ws.misc, total);
  TESS_HIP_CHECK(hipGetLastError());
  int32_t max_row = 0;
  unsigned long long pairs = 0;
  TESS_HIP_CHECK(hipMemcpyAsync(&max_row, ws.misc, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipMemcpyAsync(&pairs, total, sizeof(pairs), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipStreamSynchronize(st));
  *n_edges = (int64_t)pairs;
  if (max_row > kMaxRow) return TESS_ERR_ROW;
  // a total that row_ptr (int32) cannot hold is reported like a capacity shortfall, with the
  // true count; no edge_cap satisfies it
  if ((int64_t)pairs > edge_cap || pairs > (unsigned long long)INT32_MAX) return TESS_ERR_CAPACITY;
  TESS_TIMED("nbr_fill", st,
             k_pairs<true><<<n, 64, 0, st>>>(n, g, rcs2, pos, ws.cell_id, ws.cell_start,
                                             ws.cell_atoms, row_ptr, col_shift, ws.misc));
  TESS_HIP_CHECK(hipGetLastError());
  if (rev) {
    k_rev<<<grid(n, 4), 256, 0, st>>>(n, row_ptr, col_shift, rev);
    TESS_HIP_CHECK(hipGetLastError());
  }
  return TESS_OK;
}

}  // namespace tess
