// C ABI entry points that touch the device: build, decode, dense baseline,
// export, clone, status, free.  Argument rules are documented in include/cfr.h.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <mutex>
#include <new>
#include <string>

#include "kernels.h"

using namespace cfr;

namespace {

int hipf(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Makes the reader's device current for the scope of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = prev == dev || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// The reader's own workspace: the decode's buffers for max_batch tokens (with
// the debug copies), then the router's logits and arrival counters and the
// status word.
struct WorkspaceLayout {
  size_t decode, rlog, rarr, status, total;
  explicit WorkspaceLayout(const cfr_reader& r) {
    const cfr_config& c = r.cfg;
    auto rnd = [](size_t n) { return (n + 255) / 256 * 256; };
    size_t o = 0;
    auto take = [&](size_t bytes) {
      const size_t at = o;
      o += rnd(bytes);
      return at;
    };
    decode = take(carve_decode_workspace(r, c.max_batch, true, nullptr, nullptr, true));
    rlog = take(sizeof(float) * c.max_batch * c.n_experts);
    rarr = take(sizeof(int32_t) * c.max_batch);
    status = take(sizeof(int32_t));
    total = o;
  }
};

size_t workspace_bytes(const cfr_reader& r) { return WorkspaceLayout(r).total; }

void carve_workspace(cfr_reader& r) {
  const WorkspaceLayout l(r);
  char* p = static_cast<char*>(r.ws);
  carve_decode_workspace(r, r.cfg.max_batch, true, p + l.decode, &r.wk, true);
  r.rlog = reinterpret_cast<float*>(p + l.rlog);
  r.rarr = reinterpret_cast<int32_t*>(p + l.rarr);
  r.status = reinterpret_cast<int32_t*>(p + l.status);
}

void free_reader(cfr_reader* r) {
  if (!r) return;
  void* bufs[] = {r->w3, r->codes, r->scales, r->rho, r->norms, r->u,
                  r->b,  r->sigma, r->router, r->ws};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  delete r;
}

void init_geometry(cfr_reader& r) {
  r.nblk = r.cfg.hidden / kBlock;
  r.lp = half_bytes(r.cfg.inter);
  r.unit = unit_bytes(r.cfg.inter);
  r.ncand = r.cfg.top * r.cfg.inter;
  {
    const SelectGeom g = select_geom(r.ncand);
    r.ncp = g.nt * g.per;
  }
}

struct ResidentSizes {
  size_t w3, codes, scales, norms, u, b, sigma, router;
};

ResidentSizes resident_sizes(const cfr_reader& r) {
  const cfr_config& c = r.cfg;
  const size_t E = c.n_experts, I = c.inter, H = c.hidden;
  ResidentSizes s;
  s.w3 = E * I * 3 * (size_t)row_bytes((int)H, q4_rows(c));
  s.codes = E * r.nblk * kBlock * r.unit;
  s.scales = E * r.nblk * 2 * I * 2;
  s.norms = E * I * 4;
  s.u = H * (size_t)c.rank * 2;
  s.b = E * I * (size_t)c.rank * 2;
  s.sigma = H * 4;
  s.router = E * H * 2;
  return s;
}

int alloc_resident(cfr_reader& r, bool with_router) {
  ResidentSizes s = resident_sizes(r);
  hipError_t e;
  auto al = [&](void** p, size_t n) { return hipMalloc(p, n ? n : 256); };
  // the screen kernel reads whole dwords around its byte slice: up to 19
  // bytes past the last unit, so the codes allocation carries a tail pad
  if ((e = al((void**)&r.w3, s.w3)) != hipSuccess || (e = al((void**)&r.codes, s.codes + 64)) != hipSuccess ||
      (e = al((void**)&r.scales, s.scales)) != hipSuccess ||
      (e = al((void**)&r.rho, s.scales)) != hipSuccess ||
      (e = al((void**)&r.norms, s.norms)) != hipSuccess ||
      (e = al((void**)&r.u, s.u)) != hipSuccess || (e = al((void**)&r.b, s.b)) != hipSuccess ||
      (e = al((void**)&r.sigma, s.sigma)) != hipSuccess ||
      (with_router && (e = al((void**)&r.router, s.router)) != hipSuccess))
    return fail(CFR_ENOMEM, std::string("device allocation: ") + hipGetErrorString(e));
  r.ws_bytes = workspace_bytes(r);
  if ((e = hipMalloc(&r.ws, r.ws_bytes)) != hipSuccess)
    return fail(CFR_ENOMEM, std::string("workspace allocation: ") + hipGetErrorString(e));
  carve_workspace(r);
  // zeroed once: the screen accumulators start at zero (the reduce kernel
  // clears them after every decode) and every index a kernel can read from
  // the workspace is then valid
  if ((e = hipMemset(r.ws, 0, r.ws_bytes)) != hipSuccess) return hipf(e, "workspace init");
  return CFR_OK;
}

template <typename T>
std::unique_ptr<T[]> host_array(size_t n) {
  return std::unique_ptr<T[]>(new (std::nothrow) T[n ? n : 1]);
}

int check_decode_args(cfr_reader* r, const void* x, const void* ids, const void* gw, int batch,
                      int k, const void* y) {
  if (!r) return fail(CFR_EINVAL, "reader is NULL");
  if (!x || !ids || !gw || !y) return fail(CFR_EINVAL, "x, expert_ids, gate_w and y must be non-NULL");
  if (batch < 1 || batch > r->cfg.max_batch)
    return fail(CFR_EINVAL, "batch must be in 1..max_batch");
  if (k < 0 || k > r->ncand) return fail(CFR_EINVAL, "k must be in 0..top*inter");
  return CFR_OK;
}

// Scratch of the allocation-free decode: the decode's per-call buffers
// live in this file-scope array (each device holds its own copy, for as long
// as the library stays loaded).  Host code must not pass the array's name to
// a kernel: it is a host-side stand-in.  Its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchDevices {
  std::mutex m;
  void* ptr[kMaxDevices] = {};
  // leading bytes of the array known to be zero: the screen accumulates its
  // sums into the start of the array, whose extent depends on the call's
  // shape, and a previous call may have left hand-over words past its own sums
  size_t zero_upto[kMaxDevices] = {};
};
ScratchDevices g_scratch;

// This device's copy of scratch, with its first `sums` bytes zero: the part
// not known to be zero is cleared by a fill kernel on `st` first (the whole
// array, the first time a device is used).
int scratch_on_device(int dev, size_t sums, hipStream_t st, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(CFR_EUNSUPPORTED, "device ordinal above the scratch table");
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hipf(e, "scratch address");
    g_scratch.ptr[dev] = p;
    g_scratch.zero_upto[dev] = 0;
    sums = kScratchBytes;
  }
  const size_t z = g_scratch.zero_upto[dev];
  if (sums > z) {
    const hipError_t e = launch_zero(static_cast<char*>(g_scratch.ptr[dev]) + z, sums - z, st);
    if (e != hipSuccess) return hipf(e, "scratch clear");
  }
  *out = g_scratch.ptr[dev];
  return CFR_OK;
}

}  // namespace

extern "C" {

int cfr_reader_decode_noalloc(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                              int32_t batch, int32_t k, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  const size_t need = carve_decode_workspace(*r, batch, false, nullptr, nullptr);
  if (need > kScratchBytes)
    return fail(CFR_EUNSUPPORTED, "this call needs " + std::to_string(need) +
                                      " bytes of decode scratch, above the " + std::to_string(kScratchBytes) +
                                      " bytes of the allocation-free entry point: use cfr_reader_decode or a "
                                      "smaller batch");
  DeviceGuard guard(r->cfg.device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the screen sums come first in the carve: their extent must start zero
  const size_t acc_bytes = decode_sums_bytes(*r, batch);
  std::lock_guard<std::mutex> lock(g_scratch.m);
  void* base = nullptr;
  rc = scratch_on_device(r->cfg.device, acc_bytes, st, &base);
  if (rc) return rc;
  Workspace w;
  carve_decode_workspace(*r, batch, false, static_cast<char*>(base), &w);
  rc = launch_decode(r, x, ids, gw, batch, k, y, st, nullptr, nullptr, -1, nullptr, &w);
  // a decode leaves its sums zero and its hand-over words after them; a
  // failed one may have left partial sums
  g_scratch.zero_upto[r->cfg.device] = rc ? 0 : acc_bytes;
  return rc;
}

int cfr_build_reader(const cfr_config* cfg, const uint16_t* gate, const uint16_t* up,
                     const uint16_t* down, const uint16_t* router, cfr_reader** out) {
  clear_error();
  if (!out) return fail(CFR_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (q4_rows(*cfg)) return fail(CFR_EINVAL, "exact_bits 4: build with cfr_build_reader_q4");
  if (!gate || !up || !down) return fail(CFR_EINVAL, "gate, up and down must be non-NULL");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev)
    return fail(CFR_EINVAL, "device ordinal not available");
  DeviceGuard guard(cfg->device);
  if (!guard.ok) return fail(CFR_EHIP, "cannot select device");

  std::unique_ptr<cfr_reader, void (*)(cfr_reader*)> r(new (std::nothrow) cfr_reader(), free_reader);
  if (!r) return fail(CFR_ENOMEM, "host allocation");
  r->cfg = *cfg;
  init_geometry(*r);
  if (max_lds_needed(*cfg) > kMaxLds)
    return fail(CFR_EUNSUPPORTED, "hidden, inter and top too large for one workgroup's LDS");
  ResidentSizes s = resident_sizes(*r);

  // load steps (1), (2), (4) on the host
  auto w3 = host_array<uint16_t>(s.w3 / 2);  // BF16 rows
  auto codes = host_array<uint8_t>(s.codes);
  auto scales = host_array<uint16_t>(s.scales / 2);
  auto rho = host_array<uint16_t>(s.scales / 2);
  auto norms = host_array<float>(s.norms / 4);
  auto sigma = host_array<float>(s.sigma / 4);
  if (!w3 || !codes || !scales || !rho || !norms || !sigma)
    return fail(CFR_ENOMEM, "host staging allocation");
  rc = pack_host(*cfg, gate, up, down, codes.get(), scales.get(), rho.get(), norms.get(),
                 w3.get(), sigma.get());
  if (rc) return rc;

  rc = alloc_resident(*r, router != nullptr);
  if (rc) return rc;
  hipError_t e;
  if ((e = hipMemcpy(r->w3, w3.get(), s.w3, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->codes, codes.get(), s.codes, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->scales, scales.get(), s.scales, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->rho, rho.get(), s.scales, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->norms, norms.get(), s.norms, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->sigma, sigma.get(), s.sigma, hipMemcpyHostToDevice)) != hipSuccess ||
      (router && (e = hipMemcpy(r->router, router, s.router, hipMemcpyHostToDevice)) != hipSuccess))
    return hipf(e, "upload");
  // load step (3) on the device
  rc = device_lowrank(r.get());
  if (rc) return rc;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "build");
  *out = r.release();
  return CFR_OK;
}

int cfr_build_reader_q4(const cfr_config* cfg, const uint8_t* rows, const uint16_t* router, cfr_reader** out) {
  clear_error();
  if (!out) return fail(CFR_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!q4_rows(*cfg)) return fail(CFR_EINVAL, "cfr_build_reader_q4 takes a config with exact_bits 4");
  if (!rows) return fail(CFR_EINVAL, "rows must be non-NULL");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev)
    return fail(CFR_EINVAL, "device ordinal not available");
  DeviceGuard guard(cfg->device);
  if (!guard.ok) return fail(CFR_EHIP, "cannot select device");

  std::unique_ptr<cfr_reader, void (*)(cfr_reader*)> r(new (std::nothrow) cfr_reader(), free_reader);
  if (!r) return fail(CFR_ENOMEM, "host allocation");
  r->cfg = *cfg;
  init_geometry(*r);
  if (max_lds_needed(*cfg) > kMaxLds)
    return fail(CFR_EUNSUPPORTED, "hidden, inter and top too large for one workgroup's LDS");
  ResidentSizes s = resident_sizes(*r);
  const size_t E = cfg->n_experts, I = cfg->inter, H = cfg->hidden, rq = row_bytes((int)H, true);

  // the weights the checkpoint holds: the sketch, the norms and the recovery
  // basis are built from them, as from BF16 weights
  auto gate = host_array<float>(E * I * H);
  auto up = host_array<float>(E * I * H);
  auto down = host_array<float>(E * H * I);
  auto codes = host_array<uint8_t>(s.codes);
  auto scales = host_array<uint16_t>(s.scales / 2);
  auto rho = host_array<uint16_t>(s.scales / 2);
  auto norms = host_array<float>(s.norms / 4);
  auto sigma = host_array<float>(s.sigma / 4);
  auto drow = host_array<float>(H);
  if (!gate || !up || !down || !codes || !scales || !rho || !norms || !sigma || !drow)
    return fail(CFR_ENOMEM, "host staging allocation");
  for (size_t e = 0; e < E; ++e)
    for (size_t j = 0; j < I; ++j) {
      const uint8_t* rec = rows + (e * I + j) * 3 * rq;
      if ((rc = dequant_q4_record(rec, (int)H, gate.get() + (e * I + j) * H)) ||
          (rc = dequant_q4_record(rec + rq, (int)H, up.get() + (e * I + j) * H)) ||
          (rc = dequant_q4_record(rec + 2 * rq, (int)H, drow.get())))
        return rc;
      for (size_t h = 0; h < H; ++h) down[(e * H + h) * I + j] = drow[h];
    }
  rc = pack_host_f32(*cfg, gate.get(), up.get(), down.get(), codes.get(), scales.get(), rho.get(), norms.get(),
                     sigma.get());
  if (rc) return rc;

  rc = alloc_resident(*r, router != nullptr);
  if (rc) return rc;
  hipError_t e;
  if ((e = hipMemcpy(r->w3, rows, s.w3, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->codes, codes.get(), s.codes, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->scales, scales.get(), s.scales, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->rho, rho.get(), s.scales, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->norms, norms.get(), s.norms, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->sigma, sigma.get(), s.sigma, hipMemcpyHostToDevice)) != hipSuccess ||
      (router && (e = hipMemcpy(r->router, router, s.router, hipMemcpyHostToDevice)) != hipSuccess))
    return hipf(e, "upload");
  rc = device_lowrank(r.get());  // load step (3) from the 4-bit down rows
  if (rc) return rc;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "build");
  *out = r.release();
  return CFR_OK;
}

int cfr_reader_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                      int32_t batch, int32_t k, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  DeviceGuard guard(r->cfg.device);
  return launch_decode(r, x, ids, gw, batch, k, y, static_cast<hipStream_t>(stream), nullptr);
}

int cfr_reader_decode_residual(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                               int32_t batch, int32_t k, const float* resid, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  if (!resid) return fail(CFR_EINVAL, "resid is NULL");
  if (resid == x) return fail(CFR_EINVAL, "resid must not alias x");
  DeviceGuard guard(r->cfg.device);
  return launch_decode(r, x, ids, gw, batch, k, y, static_cast<hipStream_t>(stream), nullptr, nullptr, -1,
                       resid);
}

int cfr_reader_decode_shared(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                             int32_t batch, int32_t k, float* y, float* bscore, int32_t* kept,
                             int32_t* experts, void* stream) {
  clear_error();
  if (!r) return fail(CFR_EINVAL, "reader is NULL");
  if (!x || !ids || !gw || !y) return fail(CFR_EINVAL, "x, expert_ids, gate_w and y must be non-NULL");
  if (batch < 1 || batch > r->cfg.max_batch) return fail(CFR_EINVAL, "batch must be in 1..max_batch");
  if (batch > kMaxSharedBatch)
    return fail(CFR_EUNSUPPORTED, "the batch-shared decode takes at most 8 tokens per call");
  if (r->cfg.ranking != CFR_RANK_SCORE)
    return fail(CFR_EUNSUPPORTED, "the batch-shared decode ranks by the output-unit score only");
  if (q4_rows(r->cfg)) return fail(CFR_EUNSUPPORTED, "the batch-shared decode reads BF16 rows only");
  const int64_t nmax = (int64_t)std::min(r->cfg.n_experts, batch * r->cfg.top) * r->cfg.inter;
  if (k < 0 || k > nmax) return fail(CFR_EINVAL, "k must be in 0..min(n_experts, batch*top)*inter");
  DeviceGuard guard(r->cfg.device);
  return launch_decode_shared(r, x, ids, gw, batch, k, y, static_cast<hipStream_t>(stream), nullptr, bscore,
                              kept, experts);
}

int cfr_reader_decode_debug(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                            int32_t batch, int32_t k, float* y, float* xrot, uint8_t* sel,
                            float* ghat, float* vhat, float* score, int32_t* kept, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  DeviceGuard guard(r->cfg.device);
  DebugOut dbg;
  dbg.xrot = xrot;
  dbg.sel = sel;
  dbg.ghat = ghat;
  dbg.vhat = vhat;
  dbg.score = score;
  dbg.kept = kept;
  return launch_decode(r, x, ids, gw, batch, k, y, static_cast<hipStream_t>(stream), &dbg);
}

int cfr_reader_decode_profile(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                              int32_t batch, int32_t k, float* y, float* stage_us, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  if (!stage_us) return fail(CFR_EINVAL, "stage_us is NULL");
  DeviceGuard guard(r->cfg.device);
  hipEvent_t ev[CFR_NUM_STAGES + 1] = {};
  hipError_t e = hipSuccess;
  for (int i = 0; i <= CFR_NUM_STAGES && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (e == hipSuccess) {
    rc = launch_decode(r, x, ids, gw, batch, k, y, st, nullptr, ev);
    if (rc == CFR_OK) e = hipStreamSynchronize(st);
    for (int i = 0; i < CFR_NUM_STAGES && e == hipSuccess && rc == CFR_OK; ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[i], ev[i + 1]);
      stage_us[i] = 1000.f * ms;
    }
  }
  for (int i = 0; i <= CFR_NUM_STAGES; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  if (rc) return rc;
  if (e != hipSuccess) return hipf(e, "profile events");
  return CFR_OK;
}

int cfr_reader_decode_stage(cfr_reader* r, int32_t stage, const float* x, const int32_t* ids,
                            const float* gw, int32_t batch, int32_t k, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, k, y);
  if (rc) return rc;
  if (stage < 0 || stage >= CFR_NUM_STAGES) return fail(CFR_EINVAL, "stage out of range");
  DeviceGuard guard(r->cfg.device);
  return launch_decode(r, x, ids, gw, batch, k, y, static_cast<hipStream_t>(stream), nullptr,
                       nullptr, stage);
}

int cfr_dense_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                     int32_t batch, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, 0, y);
  if (rc) return rc;
  DeviceGuard guard(r->cfg.device);
  return launch_dense(r, x, ids, gw, batch, y, static_cast<hipStream_t>(stream));
}

int cfr_dense_decode_residual(cfr_reader* r, const float* x, const int32_t* ids, const float* gw,
                              int32_t batch, const float* resid, float* y, void* stream) {
  int rc = check_decode_args(r, x, ids, gw, batch, 0, y);
  if (rc) return rc;
  if (!resid) return fail(CFR_EINVAL, "resid is NULL");
  if (resid == x) return fail(CFR_EINVAL, "resid must not alias x");
  DeviceGuard guard(r->cfg.device);
  return launch_dense(r, x, ids, gw, batch, y, static_cast<hipStream_t>(stream), resid);
}

int cfr_reader_route(cfr_reader* r, const float* x, int32_t batch, float norm_eps, float* x_norm,
                     int32_t* expert_ids, float* gate_w, void* stream) {
  clear_error();
  if (!r) return fail(CFR_EINVAL, "reader is NULL");
  if (!x || !expert_ids || !gate_w) return fail(CFR_EINVAL, "x, expert_ids and gate_w must be non-NULL");
  if (batch < 1 || batch > r->cfg.max_batch) return fail(CFR_EINVAL, "batch must be in 1..max_batch");
  if (!r->router) return fail(CFR_EINVAL, "the reader was built without router weights");
  if (x_norm && !(norm_eps >= 0.f)) return fail(CFR_EINVAL, "norm_eps must be >= 0");
  if (x_norm == x) return fail(CFR_EINVAL, "x_norm must not alias x");
  if (route_lds_bytes(r->cfg) + 128 > kMaxLds)
    return fail(CFR_EUNSUPPORTED, "n_experts too large for the router's top-k");
  DeviceGuard guard(r->cfg.device);
  const hipError_t e = launch_route(x, r->router, r->cfg, batch, x_norm ? norm_eps : -1.f, x_norm, r->rlog,
                                    r->rarr, expert_ids, gate_w, r->status, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CFR_OK : hipf(e, "route launch");
}

int cfr_reader_export(const cfr_reader* r, uint8_t* codes, uint16_t* scales, uint16_t* rho,
                      float* norms, uint16_t* u, uint16_t* b, float* sigma) {
  clear_error();
  if (!r) return fail(CFR_EINVAL, "reader is NULL");
  DeviceGuard guard(r->cfg.device);
  ResidentSizes s = resident_sizes(*r);
  hipError_t e;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "export sync");
  auto dl = [&](void* dst, const void* src, size_t n) {
    return dst && n ? hipMemcpy(dst, src, n, hipMemcpyDeviceToHost) : hipSuccess;
  };
  if ((e = dl(codes, r->codes, s.codes)) != hipSuccess || (e = dl(scales, r->scales, s.scales)) != hipSuccess ||
      (e = dl(rho, r->rho, s.scales)) != hipSuccess || (e = dl(norms, r->norms, s.norms)) != hipSuccess ||
      (e = dl(u, r->u, s.u)) != hipSuccess || (e = dl(b, r->b, s.b)) != hipSuccess ||
      (e = dl(sigma, r->sigma, s.sigma)) != hipSuccess)
    return hipf(e, "export");
  return CFR_OK;
}

int cfr_reader_clone(const cfr_reader* src, cfr_reader** out) {
  clear_error();
  if (!src || !out) return fail(CFR_EINVAL, "src and out must be non-NULL");
  *out = nullptr;
  DeviceGuard guard(src->cfg.device);
  std::unique_ptr<cfr_reader, void (*)(cfr_reader*)> r(new (std::nothrow) cfr_reader(), free_reader);
  if (!r) return fail(CFR_ENOMEM, "host allocation");
  r->cfg = src->cfg;
  init_geometry(*r);
  int rc = alloc_resident(*r, src->router != nullptr);
  if (rc) return rc;
  ResidentSizes s = resident_sizes(*r);
  hipError_t e;
  auto cp = [&](void* dst, const void* from, size_t n) {
    return n ? hipMemcpy(dst, from, n, hipMemcpyDeviceToDevice) : hipSuccess;
  };
  if ((e = cp(r->w3, src->w3, s.w3)) != hipSuccess || (e = cp(r->codes, src->codes, s.codes)) != hipSuccess ||
      (e = cp(r->scales, src->scales, s.scales)) != hipSuccess ||
      (e = cp(r->rho, src->rho, s.scales)) != hipSuccess ||
      (e = cp(r->norms, src->norms, s.norms)) != hipSuccess || (e = cp(r->u, src->u, s.u)) != hipSuccess ||
      (e = cp(r->b, src->b, s.b)) != hipSuccess || (e = cp(r->sigma, src->sigma, s.sigma)) != hipSuccess ||
      (src->router && (e = cp(r->router, src->router, s.router)) != hipSuccess))
    return hipf(e, "clone copy");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "clone");
  *out = r.release();
  return CFR_OK;
}

int cfr_reader_config(const cfr_reader* r, cfr_config* out) {
  clear_error();
  if (!r || !out) return fail(CFR_EINVAL, "reader and out must be non-NULL");
  *out = r->cfg;
  return CFR_OK;
}

int cfr_reader_status(cfr_reader* r, int32_t* flags) {
  clear_error();
  if (!r || !flags) return fail(CFR_EINVAL, "reader and flags must be non-NULL");
  DeviceGuard guard(r->cfg.device);
  hipError_t e;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "status sync");
  if ((e = hipMemcpy(flags, r->status, sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess)
    return hipf(e, "status read");
  if ((e = hipMemset(r->status, 0, sizeof(int32_t))) != hipSuccess) return hipf(e, "status clear");
  return CFR_OK;
}

void cfr_reader_free(cfr_reader* r) {
  if (!r) return;
  DeviceGuard guard(r->cfg.device);
  (void)hipDeviceSynchronize();
  free_reader(r);
}

}  // extern "C"
