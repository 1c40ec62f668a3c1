// Argument marshalling for eager calls of tile_gather in C++.
//
// The row gather on small tables is latency-bound: a call's GPU time is a
// few microseconds, and its host time (read each tensor's pointer, shape,
// stride and dtype; build the stg_tensor descriptors; call the C entry point)
// sets how fast back-to-back eager calls run.  Through ctypes the Python
// side of that costs about 2 us, mostly in torch's per-attribute accessors;
// here the tensors are read directly.  This module only marshals: it checks
// the arguments as the ctypes binding does, fills the descriptors and calls
// libstg's tile_gather through the address the binding hands it (it does not
// link libstg).  The ctypes path stays the reference form (and records calls
// for prepare()).
#include <Python.h>

#include <c10/hip/HIPStream.h>
#include <torch/csrc/autograd/python_variable.h>

#include <cstdint>

#include "../../include/stg.h"

namespace {

using GatherFn = int (*)(const stg_tensor*, const int32_t*, int64_t, const int64_t*, const int64_t*, int32_t,
                         const stg_tensor*, void*);

int dtype_code(c10::ScalarType t) {
  switch (t) {
    case c10::ScalarType::Float: return STG_F32;
    case c10::ScalarType::BFloat16: return STG_BF16;
    case c10::ScalarType::Half: return STG_F16;
    case c10::ScalarType::Int: return STG_I32;
    case c10::ScalarType::Byte: return STG_U8;
    case c10::ScalarType::Double: return STG_F64;
    case c10::ScalarType::Long: return STG_I64;
    default: return -1;
  }
}

// the tensor behind a Python object, or null with a Python exception set
const at::Tensor* gpu_tensor(PyObject* o, const char* name) {
  if (!THPVariable_Check(o)) {
    PyErr_Format(PyExc_TypeError, "%s must be a torch tensor", name);
    return nullptr;
  }
  const at::Tensor& t = THPVariable_Unpack(o);
  if (!t.is_cuda()) {
    PyErr_Format(PyExc_ValueError, "%s must be a GPU tensor (got device %s)", name, t.device().str().c_str());
    return nullptr;
  }
  return &t;
}

bool describe(const at::Tensor& t, const char* name, stg_tensor& d) {
  const int64_t r = t.dim();
  if (r < 1 || r > 4) {
    PyErr_Format(PyExc_ValueError, "%s: rank must be 1..4", name);
    return false;
  }
  const int code = dtype_code(t.scalar_type());
  if (code < 0) {
    PyErr_Format(PyExc_TypeError, "unsupported dtype %s", c10::toString(t.scalar_type()));
    return false;
  }
  d.data = t.data_ptr();
  d.dtype = code;
  d.rank = (int32_t)r;
  const auto sz = t.sizes(), st = t.strides();
  for (int i = 0; i < 4; ++i) {
    d.shape[i] = i < r ? sz[i] : 1;
    d.stride[i] = i < r ? st[i] : 0;
  }
  return true;
}

// a tile shape or offset: a sequence of at most 4 integers, zero-padded
bool int64x4(PyObject* o, const char* name, int64_t out[4]) {
  PyObject* seq = PySequence_Fast(o, name);
  if (!seq) return false;
  const Py_ssize_t n = PySequence_Fast_GET_SIZE(seq);
  if (n > 4) {
    Py_DECREF(seq);
    PyErr_SetString(PyExc_ValueError, "a tile shape or offset has at most 4 entries");
    return false;
  }
  PyObject** items = PySequence_Fast_ITEMS(seq);
  for (int i = 0; i < 4; ++i) out[i] = 0;
  for (Py_ssize_t i = 0; i < n; ++i) {
    out[i] = PyLong_AsLongLong(items[i]);
    if (out[i] == -1 && PyErr_Occurred()) {
      Py_DECREF(seq);
      return false;
    }
  }
  Py_DECREF(seq);
  return true;
}

// tile_gather(fn, a, indices, out, tile_shape, offset, axis, stream) -> status
// fn: address of libstg's tile_gather; offset and stream may be None (stream:
// the current stream of a's device).
PyObject* tile_gather(PyObject*, PyObject* args) {
  unsigned long long fn_addr;
  PyObject *a_o, *i_o, *o_o, *ts_o, *off_o, *st_o;
  int axis;
  if (!PyArg_ParseTuple(args, "KOOOOOiO", &fn_addr, &a_o, &i_o, &o_o, &ts_o, &off_o, &axis, &st_o)) return nullptr;
  const at::Tensor* a = gpu_tensor(a_o, "a");
  if (!a) return nullptr;
  const at::Tensor* idx = gpu_tensor(i_o, "indices");
  if (!idx) return nullptr;
  const at::Tensor* out = gpu_tensor(o_o, "out");
  if (!out) return nullptr;
  if (idx->scalar_type() != c10::ScalarType::Int || !idx->is_contiguous()) {
    PyErr_SetString(PyExc_ValueError, "indices must be a contiguous torch.int32 tensor");
    return nullptr;
  }
  stg_tensor ad, od;
  if (!describe(*a, "a", ad) || !describe(*out, "out", od)) return nullptr;
  int64_t ts[4], off[4];
  if (!int64x4(ts_o, "tile_shape", ts)) return nullptr;
  const bool has_off = off_o != Py_None;
  if (has_off && !int64x4(off_o, "offset", off)) return nullptr;
  void* stream;
  if (st_o == Py_None) {
    stream = c10::hip::getCurrentHIPStream(a->get_device()).stream();
  } else {
    stream = PyLong_AsVoidPtr(st_o);
    if (!stream && PyErr_Occurred()) return nullptr;
  }
  const int rc = reinterpret_cast<GatherFn>(fn_addr)(&ad, (const int32_t*)idx->data_ptr(), idx->numel(), ts,
                                                    has_off ? off : nullptr, axis, &od, stream);
  return PyLong_FromLong(rc);
}

PyMethodDef methods[] = {
    {"tile_gather", tile_gather, METH_VARARGS, "tile_gather through libstg's entry point at the given address"},
    {nullptr, nullptr, 0, nullptr}};

PyModuleDef module = {PyModuleDef_HEAD_INIT, "_stg_fast", "C++ argument marshalling for eager tile_gather calls", -1,
                      methods};

}  // namespace

PyMODINIT_FUNC PyInit__stg_fast() { return PyModule_Create(&module); }
