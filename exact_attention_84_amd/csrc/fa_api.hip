// C ABI of the attention library: argument validation, launch parameters,
// dispatch.  Every argument is checked before any HIP call, so invalid calls
// return their status without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fa_status ok() {
  g_last_error[0] = '\0';
  return FA_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// The kernels use gfx950-only instructions (v_mfma_f32_32x32x16_bf16,
// v_cvt_pk_bf16_f32); refuse any other device.
fa_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_ARCH, "device index %d unsupported", dev);
  int state = g_arch_state[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(FA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(state, std::memory_order_relaxed);
    if (state == 2) return fail(FA_ERR_ARCH, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (state != 1) return fail(FA_ERR_ARCH, "device %d is not gfx950", dev);
  return FA_OK;
}

bool valid_head_dim(int d) { return d == 64 || d == 128; }

bool valid_scale(float s) { return isfinite(s) && s > 0.f; }

constexpr long long kMaxElems = 1LL << 40;  // sanity bound on any one tensor

int round_up(int x, int m) { return (x + m - 1) / m * m; }

int default_decode_chunk(int batch, int heads_kv, int max_cache_len) {
  // Enough workgroups to fill 256 CUs several times over, chunks of at least
  // 512 keys so the per-chunk partials stay a small fraction of the traffic.
  const long long units = (long long)batch * heads_kv;
  const long long want = 8192;
  long long splits = (want + units - 1) / (units > 0 ? units : 1);
  if (splits < 1) splits = 1;
  int chunk = (int)((max_cache_len + splits - 1) / splits);
  chunk = round_up(chunk < 512 ? 512 : chunk, fa::kDecodeTile);
  // A power-of-two chunk puts the first key of every chunk at a power-of-two
  // multiple of the cache's row stride, and those start addresses crowd the
  // same HBM channels: chunks of 1024, 2048, 4096 and 8192 keys ran 3-10 %
  // slower than the sizes between them.  Take three quarters of such a chunk.
  if (chunk >= 1024 && (chunk & (chunk - 1)) == 0) chunk = chunk / 4 * 3;
  return chunk;
}

int decode_splits(int max_cache_len, int chunk) {
  const int s = (max_cache_len + chunk - 1) / chunk;
  return s < 1 ? 1 : s;
}

}  // namespace

// Scratch of fa_fwd_decode_kvcache_noalloc: the rotated queries and the
// split partials.  Every device the library runs on holds its own copy from
// the moment the code object is loaded there until the process ends.  Host
// code never names it directly (on the host the name is only a stand-in):
// it uses the device address that scratch_address() looks up.  Nothing in it
// has to start at zero: each call writes the partial LSE of every split
// (-inf for an empty one), reads a partial O only where that LSE is finite,
// and writes the rotated queries before reading them.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up once per
// device (check_device() has validated the device index).
fa_status scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !a)
        return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      p = static_cast<char*>(a);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM";
    case FA_ERR_GQA: return "FA_ERR_GQA";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE";
    case FA_ERR_ARCH: return "FA_ERR_ARCH";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_ARG: return "FA_ERR_ARG";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

// Validation and parameter set-up shared by fa_fwd and fa_fwd_ext.  Returns
// FA_OK with *empty set when there is nothing to compute.
static fa_status fwd_setup(const void* q, const void* k, const void* v, void* o, float* lse,
                           int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                           int head_dim, float scale, int causal, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                           fa_dtype o_dtype, fa::FwdKind kind, fa::FwdParams* p, bool* empty) {
  *empty = false;
  if (!valid_head_dim(head_dim))
    return fail(FA_ERR_HEADDIM, "head_dim %d not supported (64 or 128)", head_dim);
  if (batch < 0 || heads_q <= 0 || heads_kv <= 0)
    return fail(FA_ERR_SHAPE, "batch >= 0 and heads > 0 required (batch %d, heads %d/%d)", batch,
                heads_q, heads_kv);
  if (heads_q % heads_kv)
    return fail(FA_ERR_GQA, "heads_kv %d does not divide heads_q %d", heads_kv, heads_q);
  if (!valid_scale(scale)) return fail(FA_ERR_ARG, "scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1");
  if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_DTYPE, "o_dtype %d unknown", (int)o_dtype);
  const bool varlen = cu_seqlens_q != nullptr;
  int rows_q, rows_k;
  if (varlen) {
    if (max_seqlen_q < 0 || max_seqlen_k < 0)
      return fail(FA_ERR_SHAPE, "max_seqlen_q/k must be >= 0");
    rows_q = max_seqlen_q;
    rows_k = max_seqlen_k;
  } else {
    if (seqlen_q < 0 || seqlen_k < 0) return fail(FA_ERR_SHAPE, "seqlen_q/k must be >= 0");
    rows_q = seqlen_q;
    rows_k = seqlen_k;
  }
  if ((long long)batch * rows_q * heads_q * head_dim > kMaxElems ||
      (long long)batch * rows_k * heads_kv * head_dim > kMaxElems)
    return fail(FA_ERR_SHAPE, "tensor too large");
  // the tile loads form row offsets with 24-bit multiplies
  if ((long long)heads_kv * head_dim * 2 >= (1LL << 24) ||
      (long long)heads_q * head_dim * 2 >= (1LL << 24))
    return fail(FA_ERR_SHAPE, "a token's heads span more than 16 MiB");
  // Pointers are required only for tensors that will be touched: an empty
  // tensor (no query rows, or no keys) may come with a NULL data pointer.
  if (!q || !o || !lse) {
    if ((long long)batch * rows_q > 0)
      return fail(FA_ERR_NULL, "q, o and lse must be non-NULL");
  }
  if ((!k || !v) && (long long)batch * rows_k > 0)
    return fail(FA_ERR_NULL, "k and v must be non-NULL");
  const fa::FwdPlan plan = fa::fwd_plan(kind, head_dim, causal != 0, varlen, rows_q);
  const int br = plan.block_rows;
  const long long n_qtiles = (rows_q + br - 1) / br;
  // causal query tiles are processed in pairs (heavy with light), per sequence
  const long long n_items =
      (causal && kind != fa::FwdKind::Ext) ? (n_qtiles + 1) / 2 : n_qtiles;
  const long long total = (long long)batch * heads_q * n_items;
  if (total > 0x7fffffffLL) return fail(FA_ERR_SHAPE, "too many query tiles");
  if (total == 0) {
    *empty = true;
    return ok();  // nothing to compute
  }
  p->q = static_cast<const uint16_t*>(q);
  p->k = static_cast<const uint16_t*>(k);
  p->v = static_cast<const uint16_t*>(v);
  p->o = o;
  p->lse = lse;
  p->cu_q = cu_seqlens_q;
  p->cu_k = varlen ? (cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q) : nullptr;
  p->hq = heads_q;
  p->hkv = heads_kv;
  p->group = heads_q / heads_kv;
  p->seqlen_q = seqlen_q;
  p->seqlen_k = seqlen_k;
  p->n_qtiles = (int)n_qtiles;
  p->n_items = (int)n_items;
  p->total = (int)total;
  p->waves = plan.waves;
  p->wide = plan.wide;
  p->c = scale * fa::kLog2eHost;
  p->o_f32 = o_dtype == FA_DTYPE_F32;
  const long long gs = (long long)p->group * n_items;  // <= total < 2^31
  p->fd_items = fa::FastDiv::make((uint32_t)n_items);
  p->fd_group = fa::FastDiv::make((uint32_t)p->group);
  p->fd_hkv = fa::FastDiv::make((uint32_t)heads_kv);
  p->fd_gs = fa::FastDiv::make((uint32_t)gs);
  p->remap_end = (int)((total / gs) / 8 * 8 * gs);
  return ok();
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                 int heads_q, int heads_kv, int seqlen_q, int seqlen_k, int head_dim,
                 float scale, int causal, const int32_t* cu_seqlens_q,
                 const int32_t* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                 fa_dtype o_dtype, void* stream) {
  fa::FwdParams p;
  bool empty;
  fa_status s = fwd_setup(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                          head_dim, scale, causal, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                          max_seqlen_k, o_dtype, fa::FwdKind::Plain, &p, &empty);
  if (s != FA_OK || empty) return s;
  s = check_device();
  if (s != FA_OK) return s;
  hipError_t e = fa::launch_fwd(p, head_dim, causal != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                     int head_dim, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                     fa_dtype o_dtype, void* stream) {
  if (head_dim != 128)
    return fail(FA_ERR_HEADDIM, "the FP8 forward supports head_dim 128 (got %d)", head_dim);
  if (!valid_scale(q_descale) || !valid_scale(k_descale) || !valid_scale(v_descale))
    return fail(FA_ERR_ARG, "descales must be finite and > 0");
  fa::FwdParams p;
  bool empty;
  fa_status s = fwd_setup(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                          head_dim, scale, causal, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                          max_seqlen_k, o_dtype, fa::FwdKind::Fp8, &p, &empty);
  if (s != FA_OK || empty) return s;
  const float c = scale * q_descale * k_descale * fa::kLog2eHost;
  if (!isfinite(c) || !(c > 0.f)) return fail(FA_ERR_ARG, "scale * q_descale * k_descale out of range");
  p.c = c;
  s = check_device();
  if (s != FA_OK) return s;
  hipError_t e =
      fa::launch_fwd_fp8(p, causal != 0, v_descale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "FP8 forward launch: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                     int head_dim, float scale, int causal, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                     int window_left, int window_right, float softcap,
                     const float* alibi_slopes, int alibi_batch_stride, fa_dtype o_dtype,
                     void* stream) {
  if (!(softcap >= 0.f) || softcap > 3.0e38f)
    return fail(FA_ERR_ARG, "softcap must be finite and >= 0");
  if (alibi_slopes && alibi_batch_stride != 0 && alibi_batch_stride != heads_q)
    return fail(FA_ERR_ARG, "alibi_batch_stride must be 0 or heads_q");
  fa::FwdParams p;
  bool empty;
  fa_status s = fwd_setup(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                          head_dim, scale, causal, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                          max_seqlen_k, o_dtype, fa::FwdKind::Ext, &p, &empty);
  if (s != FA_OK || empty) return s;
  s = check_device();
  if (s != FA_OK) return s;
  // Both run on the pipelined forward: a window alone on its local-window
  // instance, ALiBi or a softcap on the instance that transforms every score
  // (its online softmax then works on scores already in log2 units).
  const int left = window_left < 0 ? -1 : window_left;
  const int right = window_right < 0 ? -1 : window_right;
  hipError_t e;
  if (softcap == 0.f && !alibi_slopes) {
    e = fa::launch_fwd_local(p, head_dim, causal != 0, left, right,
                             static_cast<hipStream_t>(stream));
  } else {
    p.c = 1.f;
    e = fa::launch_fwd_xf(p, head_dim, causal != 0, left, right, scale, softcap, alibi_slopes,
                          alibi_slopes ? alibi_batch_stride : 0,
                          static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

size_t fa_decode_workspace_size(int batch, int heads_q, int max_cache_len, int head_dim,
                                int chunk) {
  if (batch < 0 || heads_q <= 0 || max_cache_len < 0 || !valid_head_dim(head_dim)) return 0;
  if (chunk < 0 || chunk % fa::kDecodeTile) return 0;
  // The default chunk depends on heads_kv, which this query does not name:
  // size for the most splits over every heads_kv that divides heads_q.
  size_t splits = 0;
  if (chunk) {
    splits = (size_t)decode_splits(max_cache_len, chunk);
  } else {
    for (int hkv = 1; hkv <= heads_q; ++hkv)
      if (heads_q % hkv == 0) {
        const size_t s = (size_t)decode_splits(max_cache_len,
                                               default_decode_chunk(batch, hkv, max_cache_len));
        splits = s > splits ? s : splits;
      }
  }
  const size_t rows = (size_t)batch * heads_q;
  return rows * splits * ((size_t)head_dim + 1) * sizeof(float);
}

fa_status fa_fwd_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_seqlens, void* o, float* lse, int batch,
                                int heads_q, int heads_kv, int max_cache_len, int head_dim,
                                float scale, int chunk, void* workspace, size_t workspace_bytes,
                                fa_dtype o_dtype, void* stream) {
  return fa_fwd_decode_kvcache(q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                               nullptr, nullptr, cache_seqlens, nullptr, 0, 0, 0, nullptr,
                               nullptr, 0, 0, 0, o, lse, batch, heads_q, heads_kv, max_cache_len,
                               head_dim, scale, chunk, workspace, workspace_bytes, o_dtype,
                               stream);
}

// Bytes of the rotated-query buffer at the start of a KV-cache decode
// workspace (256-byte aligned), when rotary is used.
static size_t qrot_bytes(int batch, int heads_q, int head_dim) {
  const size_t b = (size_t)batch * heads_q * head_dim * 2;
  return (b + 255) / 256 * 256;
}

size_t fa_decode_kvcache_workspace_size(int batch, int heads_q, int max_cache_len, int head_dim,
                                        int chunk) {
  const size_t part = fa_decode_workspace_size(batch, heads_q, max_cache_len, head_dim, chunk);
  if (part == 0) return 0;  // invalid sizes, or nothing to compute
  return qrot_bytes(batch, heads_q, head_dim) + part;
}

// The KV-cache decode step behind fa_fwd_decode_kvcache and its
// allocation-free variant.  With builtin_scratch the caller's workspace is
// ignored and the partials go to this device's copy of `scratch`.
static fa_status decode_kvcache(const void* q, void* k_cache, void* v_cache, const void* k_new,
                                const void* v_new, const int32_t* cache_seqlens,
                                const int32_t* block_table, int max_blocks_per_seq,
                                int page_size, int num_blocks, const float* rotary_cos,
                                const float* rotary_sin, int rotary_dim, int rotary_max_pos,
                                int rotary_interleaved, void* o, float* lse, int batch,
                                int heads_q, int heads_kv, int max_cache_len, int head_dim,
                                float scale, int chunk, void* workspace, size_t workspace_bytes,
                                bool builtin_scratch, fa_dtype o_dtype, void* stream) {
  // An empty batch touches no tensor: its data pointers may be NULL (as
  // those of empty torch tensors are), and there is nothing to do.
  if (batch > 0 && (!q || !k_cache || !v_cache || !cache_seqlens || !o || !lse))
    return fail(FA_ERR_NULL, "q, caches, cache_seqlens, o and lse must be non-NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(FA_ERR_NULL, "k_new and v_new must both be given or both be NULL");
  if ((rotary_cos == nullptr) != (rotary_sin == nullptr))
    return fail(FA_ERR_NULL, "rotary_cos and rotary_sin must both be given or both be NULL");
  if (!valid_head_dim(head_dim))
    return fail(FA_ERR_HEADDIM, "head_dim %d not supported (64 or 128)", head_dim);
  if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || max_cache_len < 0)
    return fail(FA_ERR_SHAPE, "batch, max_cache_len >= 0 and heads > 0 required");
  if (heads_q % heads_kv)
    return fail(FA_ERR_GQA, "heads_kv %d does not divide heads_q %d", heads_kv, heads_q);
  if (heads_q / heads_kv > fa::kDecodeMaxGroup)
    return fail(FA_ERR_SHAPE, "heads_q / heads_kv = %d exceeds %d", heads_q / heads_kv,
                fa::kDecodeMaxGroup);
  if (!valid_scale(scale)) return fail(FA_ERR_ARG, "scale must be finite and > 0");
  if (chunk < 0 || chunk % fa::kDecodeTile)
    return fail(FA_ERR_ARG, "chunk %d must be 0 or a positive multiple of %d", chunk,
                fa::kDecodeTile);
  if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_DTYPE, "o_dtype %d unknown", (int)o_dtype);
  const bool paged = block_table != nullptr;
  if (paged) {
    if (page_size <= 0 || page_size % fa::kDecodeTile)
      return fail(FA_ERR_ARG, "page_size %d must be a positive multiple of %d", page_size,
                  fa::kDecodeTile);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0)
      return fail(FA_ERR_SHAPE, "max_blocks_per_seq and num_blocks must be > 0");
    if ((long long)max_blocks_per_seq * page_size != max_cache_len)
      return fail(FA_ERR_SHAPE, "paged: max_cache_len %d must equal max_blocks_per_seq * "
                  "page_size = %lld", max_cache_len, (long long)max_blocks_per_seq * page_size);
    if ((long long)num_blocks * page_size * heads_kv * head_dim > kMaxElems)
      return fail(FA_ERR_SHAPE, "block pool too large");
  } else if ((long long)batch * max_cache_len * heads_kv * head_dim > kMaxElems) {
    return fail(FA_ERR_SHAPE, "cache too large");
  }
  const bool rot = rotary_cos != nullptr;
  if (rot && (rotary_dim <= 0 || rotary_dim % 2 || rotary_dim > head_dim || rotary_max_pos <= 0))
    return fail(FA_ERR_ARG, "rotary_dim %d must be even, in (0, head_dim], with max_pos > 0",
                rotary_dim);
  if (rotary_interleaved != 0 && rotary_interleaved != 1)
    return fail(FA_ERR_ARG, "rotary_interleaved must be 0 or 1");
  if (batch == 0) return ok();
  const int c = chunk ? chunk : default_decode_chunk(batch, heads_kv, max_cache_len);
  const int n_splits = decode_splits(max_cache_len, c);
  const size_t qrb = rot ? qrot_bytes(batch, heads_q, head_dim) : 0;
  const size_t need = qrb + fa_decode_workspace_size(batch, heads_q, max_cache_len, head_dim, c);
  if (builtin_scratch) {
    if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES)
      return fail(FA_ERR_WORKSPACE, "this call needs %zu bytes of scratch, more than the "
                  "%zu of the built-in scratch; call fa_fwd_decode_kvcache with a workspace",
                  need, (size_t)FA_NOALLOC_SCRATCH_BYTES);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) % 16)
      return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  const long long total = (long long)batch * heads_kv * n_splits;
  if (total > 0x7fffffffLL) return fail(FA_ERR_SHAPE, "too many splits");

  fa_status s = check_device();
  if (s != FA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (builtin_scratch) {
    s = scratch_address(&ws);
    if (s != FA_OK) return s;
  }

  if (rot || k_new) {
    fa::AppendParams a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.q_rot = rot ? reinterpret_cast<uint16_t*>(ws) : nullptr;
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.cache_seqlens = cache_seqlens;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.page_size = page_size;
    a.num_blocks = num_blocks;
    a.cos = rotary_cos;
    a.sin = rotary_sin;
    a.rdim = rot ? rotary_dim : 0;
    a.max_pos = rotary_max_pos;
    a.interleaved = rotary_interleaved;
    a.batch = batch;
    a.hq = heads_q;
    a.hkv = heads_kv;
    a.cache_len = max_cache_len;
    hipError_t e = fa::launch_append(a, head_dim, st);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  }

  const size_t rows = (size_t)batch * heads_q;
  fa::DecodeParams p;
  p.q = rot ? reinterpret_cast<const uint16_t*>(ws) : static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.cache_seqlens = cache_seqlens;
  p.o_part = reinterpret_cast<float*>(ws + qrb);
  p.lse_part = p.o_part + rows * n_splits * head_dim;
  p.hq = heads_q;
  p.hkv = heads_kv;
  p.group = heads_q / heads_kv;
  p.cache_len = max_cache_len;
  p.chunk = c;
  p.n_splits = n_splits;
  p.total = (int)total;
  p.c = scale * fa::kLog2eHost;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.page_size = page_size;
  p.num_blocks = num_blocks;
  p.len_add = k_new ? 1 : 0;
  hipError_t e = fa::launch_decode(p, head_dim, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  e = fa::launch_combine(p.o_part, p.lse_part, (int)rows, n_splits, head_dim, o, lse,
                         o_dtype == FA_DTYPE_F32, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_fwd_decode_kvcache(const void* q, void* k_cache, void* v_cache, const void* k_new,
                                const void* v_new, const int32_t* cache_seqlens,
                                const int32_t* block_table, int max_blocks_per_seq,
                                int page_size, int num_blocks, const float* rotary_cos,
                                const float* rotary_sin, int rotary_dim, int rotary_max_pos,
                                int rotary_interleaved, void* o, float* lse, int batch,
                                int heads_q, int heads_kv, int max_cache_len, int head_dim,
                                float scale, int chunk, void* workspace, size_t workspace_bytes,
                                fa_dtype o_dtype, void* stream) {
  return decode_kvcache(q, k_cache, v_cache, k_new, v_new, cache_seqlens, block_table,
                        max_blocks_per_seq, page_size, num_blocks, rotary_cos, rotary_sin,
                        rotary_dim, rotary_max_pos, rotary_interleaved, o, lse, batch, heads_q,
                        heads_kv, max_cache_len, head_dim, scale, chunk, workspace,
                        workspace_bytes, false, o_dtype, stream);
}

fa_status fa_fwd_decode_kvcache_noalloc(const void* q, void* k_cache, void* v_cache,
                                        const void* k_new, const void* v_new,
                                        const int32_t* cache_seqlens,
                                        const int32_t* block_table, int max_blocks_per_seq,
                                        int page_size, int num_blocks, const float* rotary_cos,
                                        const float* rotary_sin, int rotary_dim,
                                        int rotary_max_pos, int rotary_interleaved, void* o,
                                        float* lse, int batch, int heads_q, int heads_kv,
                                        int max_cache_len, int head_dim, float scale, int chunk,
                                        fa_dtype o_dtype, void* stream) {
  return decode_kvcache(q, k_cache, v_cache, k_new, v_new, cache_seqlens, block_table,
                        max_blocks_per_seq, page_size, num_blocks, rotary_cos, rotary_sin,
                        rotary_dim, rotary_max_pos, rotary_interleaved, o, lse, batch, heads_q,
                        heads_kv, max_cache_len, head_dim, scale, chunk, nullptr, 0, true,
                        o_dtype, stream);
}

fa_status fa_combine(const float* o_part, const float* lse_part, int rows, int n_splits,
                     int head_dim, void* o, float* lse, fa_dtype o_dtype, void* stream) {
  if (!o_part || !lse_part || !o || !lse)
    return fail(FA_ERR_NULL, "o_part, lse_part, o and lse must be non-NULL");
  if (!valid_head_dim(head_dim))
    return fail(FA_ERR_HEADDIM, "head_dim %d not supported (64 or 128)", head_dim);
  if (rows < 0 || n_splits < 1 || n_splits > fa::kCombineMaxSplits)
    return fail(FA_ERR_SHAPE, "rows >= 0 and 1 <= n_splits <= %d required",
                fa::kCombineMaxSplits);
  if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_DTYPE, "o_dtype %d unknown", (int)o_dtype);
  if (rows == 0) return ok();
  fa_status s = check_device();
  if (s != FA_OK) return s;
  hipError_t e = fa::launch_combine(o_part, lse_part, rows, n_splits, head_dim, o, lse,
                                    o_dtype == FA_DTYPE_F32, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

size_t fa_bwd_workspace_size(int batch, int heads_q, int max_seqlen_q) {
  if (batch < 0 || heads_q <= 0 || max_seqlen_q < 0) return 0;
  const long long rows = (long long)batch * max_seqlen_q;
  if (rows > kMaxElems) return 0;
  return 2 * (size_t)heads_q * (size_t)(rows + fa::kBwdPad) * sizeof(float);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int batch, int heads_q,
                 int heads_kv, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int max_seqlen_q,
                 int max_seqlen_k, fa_dtype grad_dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!valid_head_dim(head_dim))
    return fail(FA_ERR_HEADDIM, "head_dim %d not supported (64 or 128)", head_dim);
  if (batch < 0 || heads_q <= 0 || heads_kv <= 0)
    return fail(FA_ERR_SHAPE, "batch >= 0 and heads > 0 required (batch %d, heads %d/%d)", batch,
                heads_q, heads_kv);
  if (heads_q % heads_kv)
    return fail(FA_ERR_GQA, "heads_kv %d does not divide heads_q %d", heads_kv, heads_q);
  if (!valid_scale(scale)) return fail(FA_ERR_ARG, "scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1");
  if (grad_dtype != FA_DTYPE_BF16 && grad_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_DTYPE, "grad_dtype %d unknown", (int)grad_dtype);
  const bool varlen = cu_seqlens_q != nullptr;
  int rows_q, rows_k;
  if (varlen) {
    if (max_seqlen_q < 0 || max_seqlen_k < 0)
      return fail(FA_ERR_SHAPE, "max_seqlen_q/k must be >= 0");
    rows_q = max_seqlen_q;
    rows_k = max_seqlen_k;
  } else {
    if (seqlen_q < 0 || seqlen_k < 0) return fail(FA_ERR_SHAPE, "seqlen_q/k must be >= 0");
    rows_q = seqlen_q;
    rows_k = seqlen_k;
  }
  const long long nq = (long long)batch * rows_q, nk = (long long)batch * rows_k;
  if (nq * heads_q * head_dim > kMaxElems || nk * heads_kv * head_dim > kMaxElems)
    return fail(FA_ERR_SHAPE, "tensor too large");
  if ((!q || !o || !dout || !lse || !dq) && nq > 0)
    return fail(FA_ERR_NULL, "q, o, dout, lse and dq must be non-NULL");
  if ((!k || !v || !dk || !dv) && nk > 0)
    return fail(FA_ERR_NULL, "k, v, dk and dv must be non-NULL");
  const int bq = fa::bwd_dq_rows(), bk = fa::bwd_dkdv_keys();
  const long long n_qtiles = (rows_q + bq - 1) / bq;
  const long long n_kblocks = (rows_k + bk - 1) / bk;
  if ((long long)batch * heads_q * n_qtiles > 0x7fffffffLL ||
      (long long)batch * heads_kv * n_kblocks > 0x7fffffffLL || nq * heads_q > 0x7fffffffLL)
    return fail(FA_ERR_SHAPE, "too many tiles");
  if (nq == 0 && nk == 0) return ok();  // nothing to compute
  const size_t need = fa_bwd_workspace_size(batch, heads_q, rows_q);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3))
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes, 4-byte aligned (got %zu)", need,
                workspace_bytes);

  fa_status s = check_device();
  if (s != FA_OK) return s;

  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.rows_cap = (int)nq;
  p.ws_stride = p.rows_cap + fa::kBwdPad;
  p.dsum = static_cast<float*>(workspace);
  p.lse2 = p.dsum + (size_t)heads_q * p.ws_stride;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.cu_q = cu_seqlens_q;
  p.cu_k = varlen ? (cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q) : nullptr;
  p.batch = batch;
  p.hq = heads_q;
  p.hkv = heads_kv;
  p.group = heads_q / heads_kv;
  p.seqlen_q = seqlen_q;
  p.seqlen_k = seqlen_k;
  p.n_qtiles = (int)n_qtiles;
  p.n_kblocks = (int)n_kblocks;
  p.scale = scale;
  p.c = scale * fa::kLog2eHost;
  p.g_f32 = grad_dtype == FA_DTYPE_F32;
  hipError_t e = fa::launch_bwd(p, head_dim, causal != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
