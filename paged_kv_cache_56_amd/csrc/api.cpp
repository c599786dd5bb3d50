// C ABI of libpagedkv: argument checks on the host, then asynchronous launches.
// Nothing here touches the device before every check has passed, so the
// error paths can be exercised on a machine without a GPU.
#include "pkv_internal.h"

#include <cmath>
#include <mutex>

using namespace pkv;

// Device scratch of pkv_paged_decode_attn_noalloc: the split-context
// workspace (partial results per query row and context piece) lives here
// instead of in a caller buffer.  Each device that loads the library holds
// its own copy, zero-filled at load, until the process ends.  In host code
// `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device (scratch_of_stream below).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to, looked up
// on the first call for that device with the device current.
int scratch_of_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return PKV_ERR_LAUNCH;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    g_scratch_err[dev] = hipGetDevice(&cur);
    if (g_scratch_err[dev] != hipSuccess) return;
    if (cur != dev && (g_scratch_err[dev] = hipSetDevice(dev)) != hipSuccess) return;
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
    if (cur != dev) (void)hipSetDevice(cur);
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return PKV_ERR_LAUNCH;
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

int elem_bytes(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_INT8: return 1;
    default: return 0;
  }
}

int check_dims(const pkv_decode_dims* d) {
  if (!d) return PKV_ERR_NULL;
  if (d->num_seqs <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 || d->partition_blocks < 0 ||
      d->window < 0 || d->sinks < 0 || d->total_blocks < 0)
    return PKV_ERR_SHAPE;
  if (d->sink_tiles != 0 && d->sink_tiles != 1) return PKV_ERR_SHAPE;
  if (d->sink_tiles && (d->sinks < 1 || d->sinks > PKV_BLOCK_SIZE)) return PKV_ERR_SHAPE;
  if (d->block_size != PKV_BLOCK_SIZE) return PKV_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads) return PKV_ERR_SHAPE;
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PKV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_ERR_SHAPE;
  // grid dimensions: y = KV heads, z = sequences (HIP limits y, z to 65535)
  if (d->num_kv_heads > 65535 || d->num_seqs > 65535) return PKV_ERR_SHAPE;
  if (d->prefix_groups < 0 || d->prefix_max_seqs < 0 || d->prefix_max_blocks < 0)
    return PKV_ERR_SHAPE;
  if (d->prefix_groups > 0) {
    if (d->prefix_max_seqs < 1 || d->prefix_max_blocks > d->max_blocks_per_seq) return PKV_ERR_SHAPE;
    if (d->window != 0 || d->sink_tiles) return PKV_ERR_SHAPE;
    const int64_t z = (int64_t)d->prefix_groups * (((int64_t)d->prefix_max_seqs * g + 63) / 64);
    if (z > 65535) return PKV_ERR_SHAPE;   // grid z of the shared-prefix pass
  }
  if (!elem_bytes(d->q_dtype) || !elem_bytes(d->kv_dtype) || !elem_bytes(d->out_dtype))
    return PKV_ERR_DTYPE;
  return PKV_OK;
}

bool is_q8(int dt) { return dt == PKV_FP8_E4M3 || dt == PKV_INT8; }

// v_dtype < 0: the unquantised entry point (q, K, V, out of one float type).
int check_dtypes(const pkv_decode_dims* d, int v_dtype) {
  if (v_dtype >= 0) {
    const int k = d->kv_dtype, q = d->q_dtype, o = d->out_dtype;
    if (is_q8(q) || is_q8(o)) return PKV_ERR_DTYPE;
    if (k == PKV_F16 || k == PKV_BF16)   // 16-bit K with 8-bit V: q and out of K's type
      return is_q8(v_dtype) && q == k && o == k ? PKV_OK : PKV_ERR_DTYPE;
    if (k == PKV_FP8_E4M3 && v_dtype == PKV_FP8_E4M3) {
      const bool ok = (q == o) || (o == PKV_F32 && (q == PKV_BF16 || q == PKV_F16));
      return ok ? PKV_OK : PKV_ERR_DTYPE;
    }
    const bool pair = (k == PKV_FP8_E4M3 && v_dtype == PKV_INT8) ||
                      (k == PKV_INT8 && v_dtype == PKV_INT8);
    const bool qo = (q == PKV_BF16 || q == PKV_F16) && o == q;
    return pair && qo ? PKV_OK : PKV_ERR_DTYPE;
  }
  if (is_q8(d->kv_dtype)) return PKV_ERR_DTYPE;
  if (d->q_dtype != d->kv_dtype || d->out_dtype != d->kv_dtype) return PKV_ERR_DTYPE;
  return PKV_OK;
}

// Shared-prefix group arguments (both NULL: the entry points without groups).
struct GroupPtrs {
  const int32_t* seq_start;
  const int32_t* blocks;
};

// The step's append carried by the attention launch (pkv_paged_decode_step).
struct StepAppend {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
};

// qp: the 8-bit arguments (NULL for the f32/f16/bf16 entry points).
int decode_common(const void* q, const void* k_cache, const void* v_cache, const pkv_quant_params* qp,
                  const GroupPtrs* gp, const int32_t* block_tables, const int32_t* context_lens,
                  float scale, void* out, const pkv_decode_dims* dims, void* workspace,
                  size_t workspace_bytes, hipStream_t stream, const StepAppend* ap = nullptr,
                  bool use_scratch = false) {
  int st = check_dims(dims);
  if (st) return st;
  if (ap) {
    if (dims->sink_tiles) return PKV_ERR_SHAPE;          // no full-precision sink tiles
    if (!qp && is_q8(dims->kv_dtype)) return PKV_ERR_DTYPE;
    if (!ap->k_new || !ap->v_new || !ap->slots) return PKV_ERR_NULL;
  }
  if (!gp && dims->prefix_groups != 0) return PKV_ERR_SHAPE;   // groups: the _prefix entry point
  if (gp) {
    if (dims->prefix_groups > 0 && (!gp->seq_start || !gp->blocks)) return PKV_ERR_NULL;
    if (qp) {
      // the group pass on 8-bit caches: K and V of one 8-bit format with one
      // scale per (block, KV head), a 16-bit query and output of one type,
      // head_dim 128, no full-precision sink tiles
      if (!is_q8(dims->kv_dtype) || qp->v_dtype != dims->kv_dtype) return PKV_ERR_DTYPE;
      if (qp->k_channel_scales || qp->k_scales_per_token || qp->v_scales_per_token) return PKV_ERR_DTYPE;
      if (dims->q_dtype != dims->out_dtype || (dims->q_dtype != PKV_F16 && dims->q_dtype != PKV_BF16))
        return PKV_ERR_DTYPE;
      if (dims->head_dim != 128 || dims->sink_tiles) return PKV_ERR_SHAPE;
    } else if (dims->kv_dtype != PKV_F16 && dims->kv_dtype != PKV_BF16) {
      return PKV_ERR_DTYPE;
    }
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (qp) {
    const bool k8 = is_q8(dims->kv_dtype);
    if (!qp->v_scales || (k8 && !qp->k_scales)) return PKV_ERR_NULL;
    if (!k8 && (qp->k_scales || qp->k_channel_scales || qp->k_scales_per_token))
      return PKV_ERR_DTYPE;                    // a 16-bit K is read as stored
    if ((qp->k_scales_per_token != 0 && qp->k_scales_per_token != 1) ||
        (qp->v_scales_per_token != 0 && qp->v_scales_per_token != 1))
      return PKV_ERR_SHAPE;
  }
  if (dims->sink_tiles) {
    if (!qp) return PKV_ERR_SHAPE;            // side tiles exist for 8-bit caches only
    if (!qp->k_sink || !qp->v_sink || !qp->sink_tiles_of_seq) return PKV_ERR_NULL;
    if (qp->num_sink_tiles <= 0) return PKV_ERR_SHAPE;
  }
  const int v_dtype = qp ? qp->v_dtype : -1;
  if (qp && !is_q8(v_dtype)) return PKV_ERR_DTYPE;
  st = check_dtypes(dims, v_dtype);
  if (st) return st;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  int pb, np, gpb = 1, gnp = 0, qchunks = 0;
  plan_partitions(*dims, &pb, &np);
  if (dims->prefix_groups > 0) plan_groups(*dims, &gpb, &gnp, &qchunks);
  const size_t need = workspace_bytes_for(*dims);
  if (use_scratch) {
    if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  } else if (need && (!workspace || workspace_bytes < need)) {
    return PKV_ERR_WORKSPACE;
  }

  DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scales = qp ? qp->k_scales : nullptr;
  a.v_scales = qp ? qp->v_scales : nullptr;
  a.k_chan = qp ? qp->k_channel_scales : nullptr;
  a.k_tok = qp ? qp->k_scales_per_token : 0;
  a.v_tok = qp ? qp->v_scales_per_token : 0;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale = scale * 1.4426950408889634f;  // scores are kept in log2 units
  a.out = out;
  const size_t rows = (size_t)dims->num_seqs * dims->num_q_heads;
  a.split = need ? 1 : 0;
  a.o_part = need ? (float*)workspace : nullptr;
  a.ml_part = need ? (float*)workspace + rows * (np + gnp) * dims->head_dim : nullptr;
  a.num_seqs = dims->num_seqs;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.num_blocks = dims->num_blocks;
  a.max_blocks = dims->max_blocks_per_seq;
  a.part_blocks = pb;
  a.num_parts = np;
  a.part_stride = np + gnp;
  if (dims->prefix_groups > 0) {
    a.group_seq_start = gp->seq_start;
    a.group_blocks = gp->blocks;
    a.num_groups = dims->prefix_groups;
    a.group_max_seqs = dims->prefix_max_seqs;
    a.group_max_blocks = dims->prefix_max_blocks;
    a.group_part_blocks = gpb;
    a.group_num_parts = gnp;
    a.group_qchunks = qchunks;
    const int64_t gw = (int64_t)gnp * dims->num_kv_heads * dims->prefix_groups * qchunks;
    const int64_t dw = (int64_t)np * dims->num_kv_heads * dims->num_seqs;
    if (gw + dw > 0x7FFFFFFF) return PKV_ERR_SHAPE;   // one-dimensional grid
    a.group_wgs = (int)gw;
  }
  a.window = dims->window;
  a.sinks = (dims->window > 0 || dims->sink_tiles) ? dims->sinks : 0;
  a.sink_tiles = dims->sink_tiles;
  if (dims->sink_tiles) {
    a.sink_k = qp->k_sink;
    a.sink_v = qp->v_sink;
    a.sink_of_seq = qp->sink_tiles_of_seq;
    a.num_sink_tiles = qp->num_sink_tiles;
  }
  if (ap) {
    a.k_new = ap->k_new;
    a.v_new = ap->v_new;
    a.new_slots = ap->slots;
    a.k_cache_rw = ap->k_cache;
    a.v_cache_rw = ap->v_cache;
  }
  a.q_dtype = dims->q_dtype;
  a.kv_dtype = dims->kv_dtype;
  a.v_dtype = v_dtype >= 0 ? v_dtype : dims->kv_dtype;
  a.out_dtype = dims->out_dtype;
  if (use_scratch && need) {
    // every argument is valid: only now is the device touched
    void* ws = nullptr;
    st = scratch_of_stream(stream, &ws);
    if (st) return st;
    a.o_part = (float*)ws;
    a.ml_part = (float*)ws + rows * (np + gnp) * dims->head_dim;
  }
  return launch_decode(a, stream);
}

int check_q8_append(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t block_size, int32_t src_dtype, int32_t scale_mode) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_SHAPE;
  if (block_size != PKV_BLOCK_SIZE || head_dim % 16 || head_dim > 1024) return PKV_ERR_SHAPE;
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (scale_mode != PKV_SCALE_GIVEN && scale_mode != PKV_SCALE_FIRST_WRITE &&
      scale_mode != PKV_SCALE_PER_TOKEN)
    return PKV_ERR_SHAPE;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                  int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                  hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_SHAPE;
  if (block_size != PKV_BLOCK_SIZE) return PKV_ERR_SHAPE;
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  const int row_bytes = head_dim * elem_bytes(dtype);
  if (row_bytes % 16 || head_dim > 1024) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  const bool k_only = !v_new && !v_cache;   // a 16-bit K next to an 8-bit V
  if (!k_new || !slot_mapping || !k_cache || (!k_only && (!v_new || !v_cache))) return PKV_ERR_NULL;
  return launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens,
                          num_kv_heads, row_bytes, num_blocks, stream);
}

int pkv_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t num_blocks, int32_t block_size, int32_t src_dtype,
                      int32_t scale_mode, hipStream_t stream) {
  const int st = check_q8_append(num_tokens, num_kv_heads, head_dim, num_blocks, block_size,
                                 src_dtype, scale_mode);
  if (st) return st;
  if (scale_mode == PKV_SCALE_PER_TOKEN) return PKV_ERR_SHAPE;   // per-token: pkv_kv_append_quant
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scales || !v_scales)
    return PKV_ERR_NULL;
  const QTargetArgs tg[2] = {{k_new, k_cache, k_scales, nullptr}, {v_new, v_cache, v_scales, nullptr}};
  return launch_kv_append_q8(tg, 2, slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                             src_dtype, PKV_FP8_E4M3, scale_mode, stream);
}

int pkv_kv_append_quant(const void* x_new, const int64_t* slot_mapping, void* cache, float* scales,
                        const float* channel_scales, int32_t num_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, int32_t block_size,
                        int32_t src_dtype, int32_t cache_dtype, int32_t scale_mode,
                        hipStream_t stream) {
  const int st = check_q8_append(num_tokens, num_kv_heads, head_dim, num_blocks, block_size,
                                 src_dtype, scale_mode);
  if (st) return st;
  if (!is_q8(cache_dtype)) return PKV_ERR_DTYPE;
  if (num_tokens == 0) return PKV_OK;
  if (!x_new || !slot_mapping || !cache || !scales) return PKV_ERR_NULL;
  const QTargetArgs tg[1] = {{x_new, cache, scales, channel_scales}};
  return launch_kv_append_q8(tg, 1, slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                             src_dtype, cache_dtype, scale_mode, stream);
}

int pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                    const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t dtype,
                    hipStream_t stream) {
  if (num_pairs < 0 || num_pairs > 65535 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_SHAPE;
  const int eb = elem_bytes(dtype);
  if (!eb) return PKV_ERR_DTYPE;
  const int64_t block_bytes = (int64_t)num_kv_heads * PKV_BLOCK_SIZE * head_dim * eb;
  if (block_bytes % 16 || block_bytes > (1 << 30)) return PKV_ERR_SHAPE;
  if (is_q8(dtype) ? (!k_scales || !v_scales) : (k_scales || v_scales)) return PKV_ERR_DTYPE;
  if (is_q8(dtype) && num_kv_heads > 256) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks) return PKV_ERR_NULL;
  return launch_copy_blocks(k_cache, v_cache, k_scales, v_scales, src_blocks, dst_blocks,
                            num_pairs, num_kv_heads, (int)block_bytes, num_blocks, stream);
}

size_t pkv_decode_workspace_bytes(const pkv_decode_dims* dims) {
  if (check_dims(dims) != PKV_OK) return 0;
  return workspace_bytes_for(*dims);
}

int pkv_decode_num_partitions(const pkv_decode_dims* dims) {
  const int st = check_dims(dims);
  if (st) return st;
  int pb, np;
  plan_partitions(*dims, &pb, &np);
  return np;
}

int pkv_paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          void* out, const pkv_decode_dims* dims, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream);
}

int pkv_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, void* out, const pkv_decode_dims* dims,
                                  hipStream_t stream) {
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, scale, out,
                       dims, nullptr, 0, stream, nullptr, true);
}

int pkv_paged_decode_attn_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, const pkv_decode_dims* dims,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dims && dims->sink_tiles) return PKV_ERR_SHAPE;   // side tiles: the _quant entry point
  pkv_quant_params qp{};
  qp.k_scales = k_scales;
  qp.v_scales = v_scales;
  qp.v_dtype = PKV_FP8_E4M3;
  return decode_common(q, k_cache, v_cache, &qp, nullptr, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream);
}

int pkv_paged_decode_attn_quant(const void* q, const void* k_cache, const void* v_cache,
                                const pkv_quant_params* p, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, void* out,
                                const pkv_decode_dims* dims, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!p) return PKV_ERR_NULL;
  return decode_common(q, k_cache, v_cache, p, nullptr, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream);
}

int pkv_paged_decode_step(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                          const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, void* out,
                          const pkv_decode_dims* dims, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const StepAppend ap{k_new, v_new, slot_mapping, k_cache, v_cache};
  return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream, &ap);
}

int pkv_paged_decode_step_quant(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                const void* q, void* k_cache, void* v_cache, const pkv_quant_params* p,
                                const int32_t* block_tables, const int32_t* context_lens, float scale,
                                void* out, const pkv_decode_dims* dims, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!p) return PKV_ERR_NULL;
  const StepAppend ap{k_new, v_new, slot_mapping, k_cache, v_cache};
  return decode_common(q, k_cache, v_cache, p, nullptr, block_tables, context_lens, scale, out, dims,
                       workspace, workspace_bytes, stream, &ap);
}

int pkv_paged_decode_step_prefix(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                 const void* q, void* k_cache, void* v_cache,
                                 const int32_t* group_seq_start, const int32_t* group_prefix_blocks,
                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                 void* out, const pkv_decode_dims* dims, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const StepAppend ap{k_new, v_new, slot_mapping, k_cache, v_cache};
  const GroupPtrs gp{group_seq_start, group_prefix_blocks};
  return decode_common(q, k_cache, v_cache, nullptr, &gp, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream, &ap);
}

int pkv_paged_decode_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* group_seq_start, const int32_t* group_prefix_blocks,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, void* out, const pkv_decode_dims* dims,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const GroupPtrs gp{group_seq_start, group_prefix_blocks};
  return decode_common(q, k_cache, v_cache, nullptr, &gp, block_tables, context_lens, scale, out,
                       dims, workspace, workspace_bytes, stream);
}

int pkv_paged_decode_attn_quant_prefix(const void* q, const void* k_cache, const void* v_cache,
                                       const pkv_quant_params* p, const int32_t* group_seq_start,
                                       const int32_t* group_prefix_blocks, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, void* out,
                                       const pkv_decode_dims* dims, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (!p) return PKV_ERR_NULL;
  const GroupPtrs gp{group_seq_start, group_prefix_blocks};
  return decode_common(q, k_cache, v_cache, p, &gp, block_tables, context_lens, scale, out, dims, workspace,
                       workspace_bytes, stream);
}

int pkv_paged_decode_step_quant_prefix(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                       const void* q, void* k_cache, void* v_cache, const pkv_quant_params* p,
                                       const int32_t* group_seq_start, const int32_t* group_prefix_blocks,
                                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                                       void* out, const pkv_decode_dims* dims, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (!p) return PKV_ERR_NULL;
  const StepAppend ap{k_new, v_new, slot_mapping, k_cache, v_cache};
  const GroupPtrs gp{group_seq_start, group_prefix_blocks};
  return decode_common(q, k_cache, v_cache, p, &gp, block_tables, context_lens, scale, out, dims, workspace,
                       workspace_bytes, stream, &ap);
}

int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words,
                       hipStream_t stream) {
  if (sink_words < 1 || sink_words > 0x7FFFFFFF / 256) return PKV_ERR_SHAPE;
  if (bytes < 16) return PKV_OK;
  if (!buf || !sink) return PKV_ERR_NULL;
  return launch_hbm_read(buf, bytes, sink, sink_words, stream);
}

int pkv_paged_read_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, const pkv_decode_dims* dims, int32_t v_dtype,
                         uint32_t* sink, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->head_dim != 128 || dims->window != 0 || dims->sink_tiles || dims->prefix_groups)
    return PKV_ERR_SHAPE;
  const int eb = elem_bytes(dims->kv_dtype), veb = elem_bytes(v_dtype);
  if ((eb != 1 && eb != 2) || (veb != 1 && veb != 2) || veb > eb) return PKV_ERR_DTYPE;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return PKV_ERR_NULL;
  int pb, np;
  plan_partitions(*dims, &pb, &np);
  DecodeArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = dims->num_seqs;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.num_blocks = dims->num_blocks;
  a.max_blocks = dims->max_blocks_per_seq;
  a.part_blocks = pb;
  a.num_parts = np;
  a.kv_dtype = dims->kv_dtype;
  a.v_dtype = v_dtype;
  return launch_paged_read_probe(a, sink, stream);
}

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer argument";
    case PKV_ERR_SHAPE: return "invalid shape or size";
    case PKV_ERR_DTYPE: return "unsupported dtype combination";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_NO_BLOCKS: return "block pool exhausted";
    case PKV_ERR_SEQUENCE: return "unknown or duplicate sequence id";
    case PKV_ERR_SCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int pkv_version(void) { return PKV_VERSION; }

}  // extern "C"
