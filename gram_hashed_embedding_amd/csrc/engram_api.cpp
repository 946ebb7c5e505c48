// libengram C ABI: host-side validation and launch of the Engram stages.
// Every entry point checks its arguments before launching anything and
// returns an ENGRAM_* status; see include/engram.h for the contract.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "engram_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return ENGRAM_OK;
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction)
    return fail(ENGRAM_EUNSUPPORTED, "%s: no gfx950 code for the current device (%s)", what,
                hipGetErrorString(e));
  return fail(ENGRAM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// A table lives either in device memory or in pinned host memory that the
// runtime maps into the device's address space at its host address
// (hipHostMalloc); its rows then cross the host link on every read.
int check_table_memory(const void* p, const char* what) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // not sticky: the next launch check must not see it
    return fail(ENGRAM_EINVAL, "%s: not device memory or pinned host memory (%s)", what,
                hipGetErrorString(e));
  }
  if (a.type == hipMemoryTypeDevice) return ENGRAM_OK;
  if (a.type == hipMemoryTypeHost && a.devicePointer == p) return ENGRAM_OK;
  return fail(ENGRAM_EINVAL, "%s: memory type %d is not device memory or pinned host memory mapped at "
              "its host address", what, (int)a.type);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Deterministic Miller-Rabin for 32-bit n (bases 2, 7, 61 suffice below 4,759,123,141).
bool is_prime_u32(uint32_t n) {
  if (n < 2) return false;
  for (uint32_t p : {2u, 3u, 5u, 7u, 11u, 13u, 61u})
    if (n % p == 0) return n == p;
  uint32_t d = n - 1;
  int r = 0;
  while ((d & 1u) == 0) { d >>= 1; ++r; }
  auto mulmod = [n](uint64_t a, uint64_t b) { return (a * b) % n; };
  for (uint64_t a : {2ull, 7ull, 61ull}) {
    uint64_t x = 1, base = a % n, e = d;
    while (e) { if (e & 1) x = mulmod(x, base); base = mulmod(base, base); e >>= 1; }
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int i = 1; i < r && composite; ++i) {
      x = mulmod(x, x);
      if (x == n - 1) composite = false;
    }
    if (composite) return false;
  }
  return true;
}

int check_struct(const engram_hash_params* p) {
  if (p == nullptr) return fail(ENGRAM_EINVAL, "params is NULL");
  uint64_t expect = 0;
  for (int j = 0; j < ENGRAM_BUCKETS; ++j) {
    if (!is_prime_u32(p->prime[j]))
      return fail(ENGRAM_EINVAL, "prime[%d] = %u is not prime", j, p->prime[j]);
    for (int i = 0; i < j; ++i)
      if (p->prime[i] == p->prime[j])
        return fail(ENGRAM_EINVAL, "prime[%d] and prime[%d] are both %u", i, j, p->prime[j]);
    if (p->offset[j] != expect)
      return fail(ENGRAM_EINVAL, "offset[%d] = %llu, expected %llu (bucket ranges must tile the table)",
                  j, (unsigned long long)p->offset[j], (unsigned long long)expect);
    expect += p->prime[j];
  }
  if (p->n_rows != expect)
    return fail(ENGRAM_EINVAL, "n_rows = %llu, expected offset[23] + prime[23] = %llu",
                (unsigned long long)p->n_rows, (unsigned long long)expect);
  if (p->n_rows >= 0xFFFFFFFFull) return fail(ENGRAM_EINVAL, "n_rows must be below 0xFFFFFFFF");
  if (p->vocab_c == 0) return fail(ENGRAM_EINVAL, "vocab_c is 0");
  if (p->pad_cid >= p->vocab_c)
    return fail(ENGRAM_EINVAL, "pad_cid %u >= vocab_c %u", p->pad_cid, p->vocab_c);
  return ENGRAM_OK;
}

int check_tokens(const uint32_t* tok, const int32_t* cu, int32_t S, int64_t T) {
  if (T < 0 || S < 0) return fail(ENGRAM_EINVAL, "negative T (%lld) or S (%d)", (long long)T, S);
  if (T > 0 && S == 0) return fail(ENGRAM_EINVAL, "T = %lld tokens but S = 0 sequences", (long long)T);
  if (T > 0 && (tok == nullptr || cu == nullptr))
    return fail(ENGRAM_EINVAL, "tok or cu_seqlens is NULL");
  if (S > 0 && cu == nullptr) return fail(ENGRAM_EINVAL, "cu_seqlens is NULL");
  if (!aligned(tok, 4) || !aligned(cu, 4)) return fail(ENGRAM_EINVAL, "tok/cu_seqlens not 4-byte aligned");
  if (T > (int64_t)INT32_MAX) return fail(ENGRAM_EINVAL, "T above 2^31-1");
  return ENGRAM_OK;
}

int check_dims(int32_t H, int32_t hc) {
  if (H <= 0 || H % 64 != 0) return fail(ENGRAM_EINVAL, "H = %d must be a positive multiple of 64", H);
  if (hc < 1 || hc > 8) return fail(ENGRAM_EINVAL, "hc = %d must be in 1..8", hc);
  if ((int64_t)(hc + 1) * H > (1 << 20)) return fail(ENGRAM_EINVAL, "(hc+1)*H too large");
  return ENGRAM_OK;
}

// Host checks of engram_hash's arguments (also applied by engram_forward).
int check_hash_args(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                    const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                    const engram_hash_params* params, const uint32_t* idx) {
  int rc = check_struct(params);
  if (rc != ENGRAM_OK) return rc;
  rc = check_tokens(tok, cu_seqlens, S, T);
  if (rc != ENGRAM_OK) return rc;
  if (T > 0) {
    if (hist == nullptr || idx == nullptr || token_map == nullptr || map_len == 0)
      return fail(ENGRAM_EINVAL, "hist, idx or token_map missing");
    if (!aligned(hist, 4) || !aligned(idx, 4) || !aligned(token_map, 4))
      return fail(ENGRAM_EINVAL, "hist/idx/token_map not 4-byte aligned");
  }
  return ENGRAM_OK;
}

// Host checks of engram_gather_decode's arguments (also applied by engram_forward).
int check_gather_args(const uint32_t* idx, int64_t T, const uint8_t* codes, const uint8_t* scales,
                      uint64_t n_rows, const uint16_t* mem) {
  if (T < 0 || T > (int64_t)INT32_MAX) return fail(ENGRAM_EINVAL, "T out of range");
  if (T > 0) {
    if (!idx || !codes || !scales || !mem) return fail(ENGRAM_EINVAL, "NULL pointer");
    if (n_rows == 0 || n_rows >= 0xFFFFFFFFull) return fail(ENGRAM_EINVAL, "n_rows out of range");
    if (!aligned(idx, 4) || !aligned(codes, 16) || !aligned(scales, 8) || !aligned(mem, 16))
      return fail(ENGRAM_EINVAL, "idx 4-, codes 16-, scales 8-, mem 16-byte alignment required");
  }
  return ENGRAM_OK;
}

// Host checks of engram_project's arguments (also applied by engram_forward).
int check_project_args(const uint16_t* mem, int64_t T, const uint16_t* wkv,
                       const uint16_t* wkv_packed, int32_t H, int32_t hc, const uint16_t* kv) {
  int rc = check_dims(H, hc);
  if (rc != ENGRAM_OK) return rc;
  if (T < 0 || T > (int64_t)INT32_MAX) return fail(ENGRAM_EINVAL, "T out of range");
  if (T > 0) {
    if (!mem || !wkv || !kv) return fail(ENGRAM_EINVAL, "NULL pointer");
    if (!aligned(mem, 16) || !aligned(wkv, 16) || !aligned(kv, 16) || !aligned(wkv_packed, 16))
      return fail(ENGRAM_EINVAL, "mem, wkv, wkv_packed and kv must be 16-byte aligned");
  }
  return ENGRAM_OK;
}

// Host checks of engram_gate's arguments (also applied by engram_forward).
int check_gate_args(const uint16_t* hidden, const uint16_t* kv, const float* wqk, const uint32_t* tok,
                    int64_t T, int32_t H, int32_t hc, float eps, const float* gate_out) {
  int rc = check_dims(H, hc);
  if (rc != ENGRAM_OK) return rc;
  if (T < 0 || T > (int64_t)INT32_MAX) return fail(ENGRAM_EINVAL, "T out of range");
  if (!(eps >= 0.0f)) return fail(ENGRAM_EINVAL, "eps must be >= 0");
  if (T > 0) {
    if (!hidden || !kv || !wqk) return fail(ENGRAM_EINVAL, "NULL pointer");
    if (!aligned(hidden, 16) || !aligned(kv, 16) || !aligned(wqk, 16))
      return fail(ENGRAM_EINVAL, "hidden, kv and wqk must be 16-byte aligned");
    if (!aligned(tok, 4) || !aligned(gate_out, 4)) return fail(ENGRAM_EINVAL, "tok/gate_out misaligned");
  }
  return ENGRAM_OK;
}

// Host checks of engram_precompute's arguments (also applied by engram_forward).
int check_precompute_args(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                          const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                          const engram_hash_params* params, const uint8_t* codes,
                          const uint8_t* scales, const uint16_t* wkv, const uint16_t* wkv_packed,
                          int32_t H, int32_t hc, uint32_t flags, void* ws, size_t ws_bytes) {
  int rc = check_dims(H, hc);
  if (rc != ENGRAM_OK) return rc;
  if (flags & ~(uint32_t)ENGRAM_PRECOMPUTE_STAGE_ROWS)
    return fail(ENGRAM_EINVAL, "unknown precompute flags 0x%x", flags);
  if (T > 0) {
    const size_t need = engram_forward_workspace(T, H, hc);
    if (ws == nullptr || ws_bytes < need)
      return fail(ENGRAM_EINVAL, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if (!aligned(ws, 256)) return fail(ENGRAM_EINVAL, "workspace must be 256-byte aligned");
  }
  const engram::WorkspaceLayout w = engram::workspace_layout(ws, T > 0 ? T : 0, H, hc);
  if ((rc = check_hash_args(tok, cu_seqlens, S, T, hist, token_map, map_len, params, w.idx)) != ENGRAM_OK ||
      (rc = check_gather_args(w.idx, T, codes, scales, params->n_rows, w.mem)) != ENGRAM_OK ||
      (rc = check_project_args(w.mem, T, wkv, wkv_packed, H, hc, w.kv)) != ENGRAM_OK)
    return rc;
  return ENGRAM_OK;
}

// Enqueues hash -> gather + decode -> projection into the workspace.
// ev: NULL, or 4 events recorded before hashing, after hashing, after
// gather + decode and after the projection.
int enqueue_precompute(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                       const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                       const engram_hash_params& params, const uint8_t* codes, const uint8_t* scales,
                       const uint16_t* wkv, const uint16_t* wkv_packed, int32_t H, int32_t hc,
                       uint32_t flags, void* ws, uint32_t* err_flags, hipEvent_t* ev,
                       hipStream_t stream, const engram::TableBuckets* tb = nullptr) {
  int rc;
  auto mark = [&](int i) -> int {
    if (ev == nullptr) return ENGRAM_OK;
    return from_hip(hipEventRecord(ev[i], stream), "engram_precompute: hipEventRecord");
  };
  if ((rc = mark(0)) != ENGRAM_OK) return rc;
  const engram::WorkspaceLayout w = engram::workspace_layout(ws, T, H, hc);
  const bool stage = (flags & ENGRAM_PRECOMPUTE_STAGE_ROWS) != 0;
  const bool packed = engram::packs_rows(T, S);
  const uint32_t* slot = packed ? w.slot : nullptr;
  if (T > 0 && !packed && !stage) {
    // Small batch: one kernel hashes, gathers and decodes; events 1 and 2
    // both mark its end.
    rc = from_hip(engram::launch_hash_gather(tok, cu_seqlens, S, T, hist, token_map, map_len, params,
                                             codes, scales, w.idx, w.mem, err_flags, stream, tb),
                  "engram_precompute: hash + gather");
    if (rc != ENGRAM_OK) return rc;
    if ((rc = mark(1)) != ENGRAM_OK) return rc;
  } else if (T > 0) {
    rc = from_hip(engram::launch_hash(tok, cu_seqlens, S, T, hist, token_map, map_len, params, w.idx,
                                      err_flags, stream),
                  "engram_precompute: hash");
    if (rc != ENGRAM_OK) return rc;
    if (packed) {
      // Only live (non-DEAD) positions are decoded and projected: a DEAD
      // position passes through the gate untouched, so its k/v are never
      // read. Their mem and kv rows are packed in position order, slot[t]
      // locating position t's and live_pos[i] the position of row i; the
      // projection and the gate read the live count on the device.
      rc = from_hip(engram::launch_live_slots(tok, T, w.slot, w.live, w.live + 1, w.live_pos, stream),
                    "engram_precompute: live slots");
      if (rc != ENGRAM_OK) return rc;
    }
    if ((rc = mark(1)) != ENGRAM_OK) return rc;
    if (stage) {
      rc = from_hip(engram::launch_stage_rows(w.idx, T, codes, scales, params.n_rows, w.stage_codes,
                                              w.stage_scales, err_flags, stream, tb),
                    "engram_precompute: stage rows");
      if (rc != ENGRAM_OK) return rc;
    }
    rc = from_hip(engram::launch_gather_decode(w.idx, T, stage ? w.stage_codes : codes,
                                               stage ? w.stage_scales : scales, params.n_rows, w.mem,
                                               slot, stage, err_flags, stream, tb),
                  "engram_precompute: gather + decode");
    if (rc != ENGRAM_OK) return rc;
  } else if ((rc = mark(1)) != ENGRAM_OK) {
    return rc;
  }
  if ((rc = mark(2)) != ENGRAM_OK) return rc;
  rc = from_hip(engram::launch_project(w.mem, T, packed ? w.live : nullptr, wkv, wkv_packed, (hc + 1) * H,
                                       w.kv, stream),
                "engram_precompute: project");
  if (rc != ENGRAM_OK) return rc;
  return mark(3);
}

// Host checks of engram_gate_precomputed's arguments.
int check_gate_precomputed_args(const uint16_t* hidden, const void* ws, size_t ws_bytes,
                                const uint32_t* tok, int32_t S, int64_t T, const float* wqk,
                                int32_t H, int32_t hc, float eps, const float* gate_out) {
  int rc = check_dims(H, hc);
  if (rc != ENGRAM_OK) return rc;
  if (S < 0) return fail(ENGRAM_EINVAL, "S < 0");
  if (T > 0) {
    const size_t need = engram_forward_workspace(T, H, hc);
    if (ws == nullptr || ws_bytes < need)
      return fail(ENGRAM_EINVAL, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if (!aligned(ws, 256)) return fail(ENGRAM_EINVAL, "workspace must be 256-byte aligned");
    if (tok == nullptr) return fail(ENGRAM_EINVAL, "tok is NULL");
    if (S == 0) return fail(ENGRAM_EINVAL, "T = %lld tokens but S = 0 sequences", (long long)T);
  }
  const engram::WorkspaceLayout w = engram::workspace_layout(const_cast<void*>(ws), T > 0 ? T : 0, H, hc);
  return check_gate_args(hidden, w.kv, wqk, tok, T, H, hc, eps, gate_out);
}

int enqueue_gate_precomputed(uint16_t* hidden, const void* ws, const uint32_t* tok, int32_t S,
                             int64_t T, const float* wqk, int32_t H, int32_t hc, float eps,
                             float dot_scale, float* gate_out, hipStream_t stream) {
  const engram::WorkspaceLayout w = engram::workspace_layout(const_cast<void*>(ws), T, H, hc);
  const bool packed = engram::packs_rows(T, S);
  return from_hip(engram::launch_gate(hidden, w.kv, wqk, tok, packed ? w.slot : nullptr,
                                      packed ? w.live_pos : nullptr, packed ? w.live : nullptr, T, H,
                                      hc, eps, dot_scale, gate_out, stream),
                  "engram_gate_precomputed");
}

}  // namespace

namespace engram {

int report(int status, const char* what, hipError_t e) {
  if (e != hipSuccess) return fail(status, "%s: %s", what, hipGetErrorString(e));
  return fail(status, "%s", what);
}

int forward_impl(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                 const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                 const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                 const uint16_t* wkv, const uint16_t* wkv_packed, const float* wqk, uint16_t* hidden,
                 int32_t H, int32_t hc, float eps, float dot_scale, void* ws, size_t ws_bytes,
                 float* gate_out, uint32_t* err_flags, hipEvent_t* stage_events, hipStream_t stream) {
  // Every stage's arguments are checked before anything is enqueued.
  int rc = check_precompute_args(tok, cu_seqlens, S, T, hist, token_map, map_len, params, codes, scales,
                                 wkv, wkv_packed, H, hc, 0, ws, ws_bytes);
  if (rc != ENGRAM_OK) return rc;
  if ((rc = check_gate_precomputed_args(hidden, ws, ws_bytes, tok, S, T, wqk, H, hc, eps, gate_out)) !=
      ENGRAM_OK)
    return rc;
  rc = enqueue_precompute(tok, cu_seqlens, S, T, hist, token_map, map_len, *params, codes, scales, wkv,
                          wkv_packed, H, hc, 0, ws, err_flags, stage_events, stream);
  if (rc != ENGRAM_OK) return rc;
  rc = enqueue_gate_precomputed(hidden, ws, tok, S, T, wqk, H, hc, eps, dot_scale, gate_out, stream);
  if (rc != ENGRAM_OK) return rc;
  if (stage_events != nullptr)
    return from_hip(hipEventRecord(stage_events[4], stream), "engram_forward: hipEventRecord");
  return ok();
}

}  // namespace engram

extern "C" {

const char* engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ENGRAM_OK";
    case ENGRAM_EINVAL: return "ENGRAM_EINVAL: invalid argument";
    case ENGRAM_EHIP: return "ENGRAM_EHIP: HIP runtime error";
    case ENGRAM_EUNSUPPORTED: return "ENGRAM_EUNSUPPORTED: unsupported device or request";
    default: return "unknown engram status";
  }
}

const char* engram_last_error(void) { return g_last_error; }

int engram_abi_version(void) { return ENGRAM_ABI_VERSION; }

int engram_check_params(const engram_hash_params* params, const uint32_t* token_map_host,
                        uint32_t map_len) {
  int rc = check_struct(params);
  if (rc != ENGRAM_OK) return rc;
  if (map_len > 0 && token_map_host == nullptr) return fail(ENGRAM_EINVAL, "token_map_host is NULL");
  for (uint32_t i = 0; i < map_len; ++i)
    if (token_map_host[i] >= params->vocab_c)
      return fail(ENGRAM_EINVAL, "token_map[%u] = %u >= vocab_c %u (compressed vocabulary mismatch)",
                  i, token_map_host[i], params->vocab_c);
  return ok();
}

int engram_history_reset(uint32_t* hist, int32_t S, uint32_t pad_cid, hipStream_t stream) {
  if (S < 0) return fail(ENGRAM_EINVAL, "S < 0");
  if (S > 0 && (hist == nullptr || !aligned(hist, 4))) return fail(ENGRAM_EINVAL, "hist NULL or misaligned");
  return from_hip(engram::launch_history_reset(hist, S, pad_cid, stream), "engram_history_reset");
}

int engram_history_fork(uint32_t* dst, const uint32_t* src, int32_t S, hipStream_t stream) {
  if (S < 0) return fail(ENGRAM_EINVAL, "S < 0");
  if (S > 0 && (dst == nullptr || src == nullptr || !aligned(dst, 4) || !aligned(src, 4)))
    return fail(ENGRAM_EINVAL, "dst/src NULL or misaligned");
  if (S > 0 && dst == src) return fail(ENGRAM_EINVAL, "fork into the same buffer");
  return from_hip(engram::launch_history_copy(dst, src, S, stream), "engram_history_fork");
}

int engram_history_append(uint32_t* hist, const uint32_t* tok, const int32_t* cu_seqlens,
                          int32_t S, int64_t T, const uint32_t* token_map, uint32_t map_len,
                          uint32_t pad_cid, uint32_t* err_flags, hipStream_t stream) {
  int rc = check_tokens(tok, cu_seqlens, S, T);
  if (rc != ENGRAM_OK) return rc;
  if (S > 0 && (hist == nullptr || !aligned(hist, 4))) return fail(ENGRAM_EINVAL, "hist NULL or misaligned");
  if (T > 0 && (token_map == nullptr || map_len == 0)) return fail(ENGRAM_EINVAL, "empty token map");
  return from_hip(engram::launch_history_append(hist, tok, cu_seqlens, S, T, token_map, map_len,
                                                pad_cid, err_flags, stream),
                  "engram_history_append");
}

int engram_hash(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                const engram_hash_params* params, uint32_t* idx, uint32_t* err_flags,
                hipStream_t stream) {
  const int rc = check_hash_args(tok, cu_seqlens, S, T, hist, token_map, map_len, params, idx);
  if (rc != ENGRAM_OK) return rc;
  return from_hip(engram::launch_hash(tok, cu_seqlens, S, T, hist, token_map, map_len, *params,
                                      idx, err_flags, stream),
                  "engram_hash");
}

int engram_gather_decode(const uint32_t* idx, int64_t T, const uint8_t* codes,
                         const uint8_t* scales, uint64_t n_rows, uint16_t* mem,
                         uint32_t* err_flags, hipStream_t stream) {
  const int rc = check_gather_args(idx, T, codes, scales, n_rows, mem);
  if (rc != ENGRAM_OK) return rc;
  return from_hip(engram::launch_gather_decode(idx, T, codes, scales, n_rows, mem, nullptr, false, err_flags,
                                                stream),
                  "engram_gather_decode");
}

int engram_project(const uint16_t* mem, int64_t T, const uint16_t* wkv, const uint16_t* wkv_packed,
                   int32_t H, int32_t hc, uint16_t* kv, hipStream_t stream) {
  const int rc = check_project_args(mem, T, wkv, wkv_packed, H, hc, kv);
  if (rc != ENGRAM_OK) return rc;
  return from_hip(engram::launch_project(mem, T, nullptr, wkv, wkv_packed, (hc + 1) * H, kv, stream),
                  "engram_project");
}

int engram_pack_wkv(const uint16_t* wkv, int32_t H, int32_t hc, uint16_t* wkv_packed,
                    hipStream_t stream) {
  const int rc = check_dims(H, hc);
  if (rc != ENGRAM_OK) return rc;
  if (!wkv || !wkv_packed) return fail(ENGRAM_EINVAL, "NULL pointer");
  if (!aligned(wkv, 16) || !aligned(wkv_packed, 16))
    return fail(ENGRAM_EINVAL, "wkv and wkv_packed must be 16-byte aligned");
  const size_t bytes = (size_t)(hc + 1) * (size_t)H * ENGRAM_MEM * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(wkv), b = reinterpret_cast<uintptr_t>(wkv_packed);
  if (a < b + bytes && b < a + bytes) return fail(ENGRAM_EINVAL, "wkv and wkv_packed overlap");
  return from_hip(engram::launch_pack_wkv(wkv, (hc + 1) * H, wkv_packed, stream), "engram_pack_wkv");
}

int engram_gate(uint16_t* hidden, const uint16_t* kv, const float* wqk, const uint32_t* tok,
                int64_t T, int32_t H, int32_t hc, float eps, float dot_scale, float* gate_out,
                hipStream_t stream) {
  const int rc = check_gate_args(hidden, kv, wqk, tok, T, H, hc, eps, gate_out);
  if (rc != ENGRAM_OK) return rc;
  return from_hip(engram::launch_gate(hidden, kv, wqk, tok, nullptr, nullptr, nullptr, T, H, hc, eps,
                                      dot_scale, gate_out, stream),
                  "engram_gate");
}

size_t engram_forward_workspace(int64_t T, int32_t H, int32_t hc) {
  if (T <= 0 || H <= 0 || hc <= 0) return 0;
  return engram::workspace_layout(nullptr, T, H, hc).bytes;
}

int engram_precompute(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                      const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                      const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                      const uint16_t* wkv, const uint16_t* wkv_packed, int32_t H, int32_t hc,
                      uint32_t flags, void* ws, size_t ws_bytes, uint32_t* err_flags,
                      hipStream_t stream) {
  const int rc = check_precompute_args(tok, cu_seqlens, S, T, hist, token_map, map_len, params, codes,
                                       scales, wkv, wkv_packed, H, hc, flags, ws, ws_bytes);
  if (rc != ENGRAM_OK) return rc;
  return enqueue_precompute(tok, cu_seqlens, S, T, hist, token_map, map_len, *params, codes, scales,
                            wkv, wkv_packed, H, hc, flags, ws, err_flags, nullptr, stream);
}

int engram_precompute_buckets(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                              const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                              const engram_hash_params* params, const engram_bucket_table* table,
                              const uint16_t* wkv, const uint16_t* wkv_packed, int32_t H, int32_t hc,
                              uint32_t flags, void* ws, size_t ws_bytes, uint32_t* err_flags,
                              hipStream_t stream) {
  if (table == nullptr) return fail(ENGRAM_EINVAL, "table is NULL");
  engram::TableBuckets tb;
  for (int j = 0; j < ENGRAM_BUCKETS; ++j) {
    if (T > 0 && (table->codes[j] == nullptr || table->scales[j] == nullptr))
      return fail(ENGRAM_EINVAL, "bucket %d: codes or scales is NULL", j);
    if (!aligned(table->codes[j], 16) || !aligned(table->scales[j], 8))
      return fail(ENGRAM_EINVAL, "bucket %d: codes 16-byte and scales 8-byte alignment required", j);
    tb.codes[j] = reinterpret_cast<uint64_t>(table->codes[j]);
    tb.scales[j] = reinterpret_cast<uint64_t>(table->scales[j]);
  }
  // the gather's own checks see bucket 0's pointers as the table
  const int rc = check_precompute_args(tok, cu_seqlens, S, T, hist, token_map, map_len, params,
                                       table->codes[0], table->scales[0], wkv, wkv_packed, H, hc,
                                       flags, ws, ws_bytes);
  if (rc != ENGRAM_OK) return rc;
  for (int j = 0; j < ENGRAM_BUCKETS; ++j) {
    tb.first[j] = (uint32_t)params->offset[j];
    tb.count[j] = params->prime[j];
  }
  return enqueue_precompute(tok, cu_seqlens, S, T, hist, token_map, map_len, *params, nullptr, nullptr,
                            wkv, wkv_packed, H, hc, flags, ws, err_flags, nullptr, stream, &tb);
}

int engram_gate_precomputed(uint16_t* hidden, const void* ws, size_t ws_bytes, const uint32_t* tok,
                            int32_t S, int64_t T, const float* wqk, int32_t H, int32_t hc,
                            float eps, float dot_scale, float* gate_out, hipStream_t stream) {
  const int rc = check_gate_precomputed_args(hidden, ws, ws_bytes, tok, S, T, wqk, H, hc, eps, gate_out);
  if (rc != ENGRAM_OK) return rc;
  return enqueue_gate_precomputed(hidden, ws, tok, S, T, wqk, H, hc, eps, dot_scale, gate_out, stream);
}

int engram_forward(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                   const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                   const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                   const uint16_t* wkv, const uint16_t* wkv_packed, const float* wqk,
                   uint16_t* hidden, int32_t H, int32_t hc, float eps, float dot_scale, void* ws,
                   size_t ws_bytes, float* gate_out, uint32_t* err_flags,
                   hipEvent_t* stage_events, hipStream_t stream) {
  return engram::forward_impl(tok, cu_seqlens, S, T, hist, token_map, map_len, params, codes, scales,
                              wkv, wkv_packed, wqk, hidden, H, hc, eps, dot_scale, ws, ws_bytes,
                              gate_out, err_flags, stage_events, stream);
}

int engram_gen_table(uint8_t* codes, uint8_t* scales, uint64_t row_begin, uint64_t n_rows,
                     uint64_t key_data, uint64_t key_scale, hipStream_t stream) {
  if (n_rows > 0) {
    if (!codes || !scales) return fail(ENGRAM_EINVAL, "NULL pointer");
    if (!aligned(codes, 16) || !aligned(scales, 8))
      return fail(ENGRAM_EINVAL, "codes 16-byte and scales 8-byte alignment required");
    const int rc_c = check_table_memory(codes, "codes");
    if (rc_c != ENGRAM_OK) return rc_c;
    const int rc_s = check_table_memory(scales, "scales");
    if (rc_s != ENGRAM_OK) return rc_s;
  }
  return from_hip(engram::launch_gen_table(codes, scales, row_begin, n_rows, key_data, key_scale, stream),
                  "engram_gen_table");
}

}  // extern "C"
