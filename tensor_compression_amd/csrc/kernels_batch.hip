// Paged ragged batches: every sequence is coded on its own (KVTC "How the
// Pipeline Works": regions and sections are per sequence) into a container
// identical to what a contiguous call writes for it; one launch per phase
// covers the whole batch with blockIdx.z selecting the sequence.
//
// Kernels here: the per-sequence set-up (lengths, page table and workspace
// placement, validated on the device), the placement of the sequence
// containers in the batch container once their sizes are known, the copy of
// each sequence's staged fixed part, and the merge of the per-sequence status
// words into the batch status.
#include "kvtc_internal.h"

namespace kvtc {

namespace {

__device__ inline uint32_t* seq_status(const Params& p0, const SeqInfo& si) {
  return reinterpret_cast<uint32_t*>(p0.ws + si.ws_off);  // status sits at offset 0 of a workspace
}

// Block-wide exclusive scan of one value per thread (1024 threads).
__device__ inline int64_t block_exclusive_scan(int64_t v, int64_t* s_tmp, int64_t& total) {
  const int tid = threadIdx.x;
  s_tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t a = tid >= o ? s_tmp[tid - o] : 0;
    __syncthreads();
    s_tmp[tid] += a;
    __syncthreads();
  }
  total = s_tmp[1023];
  const int64_t ex = s_tmp[tid] - v;
  __syncthreads();
  return ex;
}

}  // namespace

// Clears the batch status block (k_seq_check reports into word 3).
__global__ void k_batch_clear(const Params p0) {
  if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(p0.ws)[threadIdx.x] = 0u;
}

// One workgroup per sequence: its length and every page index it uses.
__global__ __launch_bounds__(256) void k_seq_check(const Params p0, const int32_t* seq_lens, int32_t max_t_host) {
  const int z = blockIdx.x;
  const int32_t T = seq_lens[z];
  uint32_t* bst = reinterpret_cast<uint32_t*>(p0.ws);
  const int32_t np = (T + kPageTokens - 1) / kPageTokens;
  if (T < 0 || T > max_t_host || np > p0.max_pages) {
    if (threadIdx.x == 0) atomicOr(bst + 3, 1u);
    return;
  }
  const int32_t* row = p0.page_table + (int64_t)z * p0.max_pages;
  bool bad = false;
  for (int i = threadIdx.x; i < np; i += 256) bad |= row[i] < 0 || row[i] >= p0.pool_pages;
  if (bad) atomicOr(bst + 3, 1u);
}

// mode 0 (encode): lengths and page table checked, workspaces placed, status
// words cleared.  mode 1 (decode): the same, plus the batch container header
// checked and each sequence's container located.  Anything inconsistent with
// what the host sized the launches for turns every sequence empty and sets an
// error bit in the batch status, so no later kernel reads or writes outside
// its buffers.
__global__ __launch_bounds__(1024) void k_seq_setup(const Params p0, const int32_t* seq_lens, int64_t sum_t_host,
                                                    int32_t max_t_host, int64_t ws_bytes, int mode) {
  __shared__ int64_t s_tmp[1024];
  __shared__ int s_bad, s_corrupt;
  const int tid = threadIdx.x, n = p0.n_seqs;
  SeqInfo* si = reinterpret_cast<SeqInfo*>(p0.ws + batch_seqinfo_off());
  uint32_t* bst = reinterpret_cast<uint32_t*>(p0.ws);
  if (tid == 0) { s_bad = bst[3] != 0u; s_corrupt = 0; }  // k_seq_check's verdict on lengths and pages
  __syncthreads();
  int64_t sum_t = 0;
  for (int z = tid; z < n; z += 1024) sum_t += seq_lens[z];
  int64_t tot_t;
  (void)block_exclusive_scan(sum_t, s_tmp, tot_t);
  if (tid == 0 && tot_t != sum_t_host) s_bad = 1;
  // decode: the batch container header
  if (mode == 1) {
    const uint8_t* in = p0.in;
    const int64_t hb = batch_header_bytes(n);
    if (tid == 0) {
      if (p0.cap < hb) {  // too short to hold the header: read nothing
        s_corrupt = 1;
      } else {
        const uint32_t* h = reinterpret_cast<const uint32_t*>(in);
        const uint64_t total = *reinterpret_cast<const uint64_t*>(in + 16);
        if (h[0] != 0x4254564bu /* "KVTB" */ || h[1] != 1u || h[2] != (uint32_t)n || h[3] != (uint32_t)hb ||
            total > (uint64_t)p0.cap || total < (uint64_t)hb)
          s_corrupt = 1;
      }
    }
    __syncthreads();
    if (!s_corrupt) {
      const uint64_t total = *reinterpret_cast<const uint64_t*>(in + 16);
      for (int z = tid; z < n; z += 1024) {
        const uint64_t off = *reinterpret_cast<const uint64_t*>(in + kBatchFixedBytes + 16 * z);
        const uint64_t size = *reinterpret_cast<const uint64_t*>(in + kBatchFixedBytes + 16 * z + 8);
        const uint64_t prev_end = z == 0 ? (uint64_t)hb
                                         : *reinterpret_cast<const uint64_t*>(in + kBatchFixedBytes + 16 * (z - 1)) +
                                               *reinterpret_cast<const uint64_t*>(in + kBatchFixedBytes + 16 * (z - 1) + 8);
        if ((off & 255u) || off < prev_end || size < (uint64_t)kHeaderBytes || size > total || off > total - size)
          s_corrupt = 1;
      }
    }
  }
  __syncthreads();
  const bool corrupt = s_corrupt != 0;
  bool empty = s_bad != 0 || corrupt;  // every sequence coded as empty
  // workspaces, in sequence order after the batch head; when the lengths do
  // not fit the workspace the host sized, every sequence is made empty (the
  // empty layout is the smallest, so that always fits)
  const int64_t head = batch_ws_head(n);
  for (int pass = 0; pass < 2; ++pass) {
    int64_t need_total = 0;
    for (int z0 = 0; z0 < n; z0 += 1024) {
      const int z = z0 + tid;
      const int32_t T = (z < n && !empty) ? seq_lens[z] : 0;
      const int64_t need = z < n ? align256(make_ws_layout(p0.cfg, make_layout(p0.cfg, T), true).total) : 0;
      int64_t part;
      const int64_t ex = block_exclusive_scan(need, s_tmp, part);
      if (pass == 1 && z < n) {
        SeqInfo v;
        v.T = T;
        v.pad = 0;
        v.ws_off = head + need_total + ex;
        if (mode == 1 && !corrupt) {
          v.out_off = (int64_t)*reinterpret_cast<const uint64_t*>(p0.in + kBatchFixedBytes + 16 * z);
          v.cap = empty ? 0 : (int64_t)*reinterpret_cast<const uint64_t*>(p0.in + kBatchFixedBytes + 16 * z + 8);
        } else {
          v.out_off = 0;
          v.cap = mode == 0 ? ((int64_t)1 << 62) : 0;  // encode: the batch capacity is checked at placement
        }
        si[z] = v;
      }
      need_total += part;
    }
    if (pass == 0 && head + need_total > ws_bytes) {
      empty = true;
      if (tid == 0) s_bad = 1;
    }
  }
  __syncthreads();
  if (mode == 0) {
    for (int z = tid; z < n; z += 1024) {
      uint32_t* st = reinterpret_cast<uint32_t*>(p0.ws + si[z].ws_off);
      st[0] = 0; st[1] = 0; st[2] = 0; st[3] = 0;
    }
    for (int i = tid; i < n * kCountSlots; i += 1024)
      *reinterpret_cast<uint32_t*>(p0.ws + si[i / kCountSlots].ws_off + kCountOff + kCountStride * (i % kCountSlots)) = 0u;
  }
  if (tid == 0) {
    bst[0] = (s_bad ? (1u << KVTC_ERR_INVALID_ARG) : 0u) | (corrupt ? (1u << KVTC_ERR_CORRUPT) : 0u);
    bst[1] = 0; bst[2] = 0; bst[3] = 0;
  }
}

// Encode: place the sequence containers (256-byte aligned, in order, after
// the batch header) and write the batch header; on any error or overflow mark
// every sequence so that nothing is copied.
__global__ __launch_bounds__(1024) void k_batch_place(const Params p0) {
  __shared__ int64_t s_tmp[1024];
  __shared__ uint32_t s_err;
  const int tid = threadIdx.x, n = p0.n_seqs;
  SeqInfo* si = reinterpret_cast<SeqInfo*>(p0.ws + batch_seqinfo_off());
  uint32_t* bst = reinterpret_cast<uint32_t*>(p0.ws);
  if (tid == 0) s_err = bst[0];
  __syncthreads();
  const uint32_t errmask = (1u << KVTC_ERR_NONFINITE) | (1u << KVTC_ERR_CAPACITY) | (1u << KVTC_ERR_INVALID_ARG) |
                           (1u << KVTC_ERR_CORRUPT);
  const int64_t hb = batch_header_bytes(n);
  int64_t base = hb;
  for (int z0 = 0; z0 < n; z0 += 1024) {
    const int z = z0 + tid;
    int64_t size = 0;
    if (z < n) {
      const uint32_t* st = seq_status(p0, si[z]);
      if (st[0] & errmask) atomicOr(&s_err, st[0] & errmask);
      size = (int64_t)*reinterpret_cast<const uint64_t*>(st + 2);
    }
    int64_t part;
    const int64_t ex = block_exclusive_scan(align256(size), s_tmp, part);
    if (z < n) si[z].out_off = base + ex;
    base += part;
  }
  __syncthreads();
  // the batch ends with the last container (no padding after it)
  const int64_t total =
      n > 0 ? si[n - 1].out_off + (int64_t)*reinterpret_cast<const uint64_t*>(seq_status(p0, si[n - 1]) + 2) : base;
  if (!s_err && total > p0.cap) s_err = 1u << KVTC_ERR_CAPACITY;
  __syncthreads();
  const uint32_t err = s_err;
  if (err) {
    for (int z = tid; z < n; z += 1024) atomicOr(seq_status(p0, si[z]), err | (1u << KVTC_ERR_CAPACITY));
    if (tid == 0) {
      bst[0] = err;
      *reinterpret_cast<uint64_t*>(bst + 2) = 0;
    }
    return;
  }
  uint8_t* out = p0.out;
  for (int i = tid; i < hb / 4; i += 1024) {
    uint32_t v = 0;
    if (i == 0) v = 0x4254564bu;  // "KVTB"
    else if (i == 1) v = 1u;
    else if (i == 2) v = (uint32_t)n;
    else if (i == 3) v = (uint32_t)hb;
    else if (i == 4) v = (uint32_t)total;
    else if (i == 5) v = (uint32_t)((uint64_t)total >> 32);
    else if (i >= kBatchFixedBytes / 4 && i < kBatchFixedBytes / 4 + 4 * n) {
      const int z = (i - kBatchFixedBytes / 4) / 4, k = (i - kBatchFixedBytes / 4) % 4;
      const uint64_t off = (uint64_t)si[z].out_off;
      const uint64_t size = *reinterpret_cast<const uint64_t*>(seq_status(p0, si[z]) + 2);
      v = k == 0 ? (uint32_t)off : k == 1 ? (uint32_t)(off >> 32) : k == 2 ? (uint32_t)size : (uint32_t)(size >> 32);
    }
    reinterpret_cast<uint32_t*>(out)[i] = v;
  }
  // zero the alignment gap after each sequence container
  for (int z = 0; z < n; ++z) {
    const int64_t end = si[z].out_off + (int64_t)*reinterpret_cast<const uint64_t*>(seq_status(p0, si[z]) + 2);
    const int64_t next = z + 1 < n ? si[z + 1].out_off : total;
    for (int64_t i = end + tid; i < next; i += 1024) out[i] = 0;
  }
  if (tid == 0) *reinterpret_cast<uint64_t*>(bst + 2) = (uint64_t)total;
}

// Encode: a sequence's staged fixed part (header, section records, raw
// regions, directory) to its place in the batch container.
__global__ __launch_bounds__(256) void k_copy_fixed(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  if (get_status(p.ws, p.w) & ((1u << KVTC_ERR_CAPACITY) | (1u << KVTC_ERR_NONFINITE))) return;
  const int64_t units = p.chunks_off / 16;
  const uint4* src = reinterpret_cast<const uint4*>(p.ws + p.w.fixed);
  uint4* dst = reinterpret_cast<uint4*>(p.out_final);
  const int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + 256 * k;
    if (i < units) v[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + 256 * k;
    if (i < units) dst[i] = v[k];
  }
}

// Both directions: merge the sequences' status bits and exact re-computation
// counts into the batch status block.
__global__ __launch_bounds__(1024) void k_batch_finish(const Params p0) {
  const int tid = threadIdx.x, n = p0.n_seqs;
  const SeqInfo* si = reinterpret_cast<const SeqInfo*>(p0.ws + batch_seqinfo_off());
  uint32_t* bst = reinterpret_cast<uint32_t*>(p0.ws);
  uint32_t bits = 0, refined = 0;
  for (int z = tid; z < n; z += 1024) {
    const uint32_t* st = reinterpret_cast<const uint32_t*>(p0.ws + si[z].ws_off);
    bits |= st[0];
    refined += st[1];
  }
  for (int i = tid; i < n * kCountSlots; i += 1024)
    refined += *reinterpret_cast<const uint32_t*>(p0.ws + si[i / kCountSlots].ws_off + kCountOff +
                                                  kCountStride * (i % kCountSlots));
  __shared__ uint32_t s_bits, s_ref;
  if (tid == 0) { s_bits = 0; s_ref = 0; }
  __syncthreads();
  if (bits) atomicOr(&s_bits, bits);
  if (refined) atomicAdd(&s_ref, refined);
  __syncthreads();
  if (tid == 0) {
    bst[0] |= s_bits;
    bst[1] = s_ref;
    if (bst[0]) *reinterpret_cast<uint64_t*>(bst + 2) = 0;
  }
}

hipError_t launch_seq_setup(const Params& p, const int32_t* seq_lens, int64_t sum_t, int32_t max_t, int64_t ws_bytes,
                            int mode, hipStream_t s) {
  hipLaunchKernelGGL(k_batch_clear, dim3(1), dim3(64), 0, s, p);
  hipLaunchKernelGGL(k_seq_check, dim3(p.n_seqs), dim3(256), 0, s, p, seq_lens, max_t);
  hipLaunchKernelGGL(k_seq_setup, dim3(1), dim3(1024), 0, s, p, seq_lens, sum_t, max_t, ws_bytes, mode);
  return hipGetLastError();
}

hipError_t launch_batch_place(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(k_batch_place, dim3(1), dim3(1024), 0, s, p);
  const int64_t units = p.chunks_off / 16;  // the largest sequence's fixed part
  hipLaunchKernelGGL(k_copy_fixed, dim3((unsigned)((units + 1023) / 1024), 1, seq_grid(p)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_batch_finish(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(k_batch_finish, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvtc
